// The generic decode kernel: any head size that is a multiple of 32 up to
// 256, every scale mode, contiguous or paged, plain or recent-window caches,
// decode rows or chunk rows.  Included by kvq_decode.hip (head dims 32, 64,
// 128, 256) and kvq_decode_wide.hip (96, 160, 192, 224), so the
// instantiations compile in parallel.
#pragma once

#include "kvq_decode_stream.hpp"

namespace kvq {
namespace {

// ---------------------------------------------------------------------------
// Generic kernel (any supported head_dim): fp32 FMAs on codes widened in
// registers, per-lane online softmax, partials merged by decode_merge_kernel.
// On a hybrid cache a second loop takes the bf16 ring rows of the split.
// ---------------------------------------------------------------------------
template <int D, int HPW, int SM, bool PAGED>
__global__ __launch_bounds__(kThreads) void decode_generic_kernel(DecodeParams p) {
  constexpr bool G32 = SM == kSmGroup32;
  constexpr bool FP8 = SM == kSmFp8E4M3 || SM == kSmFp8E5M2;  // values, no scales
  constexpr bool E5 = SM == kSmFp8E5M2;
  // per-channel block scales: each element dequantized with its block's
  // scale for its index, (c - 128) s_d, before the dot products
  constexpr bool CH = SM == kSmBlockChannel;
  // A token row is read by NSUB lanes, 16 bytes each, in a group of LPT
  // lanes (the power of two at or above NSUB; at head dims 96, 160, 192 and
  // 224 the group's last lanes hold zeros)
  constexpr int NSUB = D / 16;
  constexpr int LPT = NSUB <= 2 ? NSUB : (NSUB <= 4 ? 4 : (NSUB <= 8 ? 8 : 16));
  constexpr int TPW = kWave / LPT;     // token rows per wave pass
  constexpr int TPP = TPW * kWaves;    // token rows per workgroup pass
  constexpr int U = 4;                 // passes issued together

  __shared__ float sm_o[kWaves][HPW][D];
  __shared__ float sm_m[kWaves][HPW];
  __shared__ float sm_l[kWaves][HPW];

  const int hg = blockIdx.x;
  const int split = blockIdx.y;
  const int v = blockIdx.z;  // the launch never sets longest_first for this kernel
  int b, qi;
  const int L = row_len(p, v, b, qi);
  const int nq = p.chunk_n > 0 ? p.chunk_n : 1;
  const int kvh = hg / p.wg_per_kvh;
  const int H = p.num_heads;
  const int h0 = kvh * (H / p.geom.kvh) + (hg % p.wg_per_kvh) * HPW;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int sub = lane % LPT;
  const int slot = lane / LPT;
  const bool sub_ok = sub < NSUB;
  const int subc = sub_ok ? sub : NSUB - 1;  // (loads of the surplus lanes stay inside the row)
  auto zero_if_off = [&](uint4 v) { return sub_ok ? v : make_uint4(0u, 0u, 0u, 0u); };

  // recent window: positions from L8 on are bf16 rows in the ring
  const int L8 = ring_start(p, b, L);
  const int t_lo = p.window > 0 ? max(L - p.window, 0) : 0;  // first visible key
  const int t_begin = t_lo + split * p.split_len;
  const int nsg = split_count(L - t_lo, p.split_len);
  if (split >= nsg) return;
  const int t_end = split == nsg - 1 ? L : t_begin + p.split_len;  // the last split takes the remainder
  const int t8_end = min(t_end, L8);  // INT8 tokens of this split end here
  const int npass = t8_end > t_begin ? (t8_end - t_begin + TPP - 1) / TPP : 0;

  float q[HPW][16];
  float qsum[HPW];
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    const uint4* qp =
        reinterpret_cast<const uint4*>(p.q + ((static_cast<int64_t>(b) * H + h0 + j) * nq + qi) * D + subc * 16);
    bf16x8_to_f32(zero_if_off(qp[0]), &q[j][0]);
    bf16x8_to_f32(zero_if_off(qp[1]), &q[j][8]);
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) s += q[j][e];
    qsum[j] = s;
  }
  const int grp = G32 ? (subc * 16) / 32 : 0;

  float m[HPW], l[HPW], ws[HPW], o[HPW][16];
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.0f;
    ws[j] = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) o[j][e] = 0.0f;
  }

  for (int ip = 0; ip < npass; ip += U) {
    uint4 kb[U], vb[U];
    float ks[U], vs[U];
    int64_t rowu[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // unconditional loads from a clamped row; out-of-range tokens are
      // discarded through their -inf score
      const int t = t_begin + (ip + u) * TPP + wave * TPW + slot;
      ok[u] = t < t8_end;
      const int tc = min(t, t8_end - 1);
      int64_t row;
      if constexpr (PAGED) {
        int phys = p.geom.block_table[static_cast<int64_t>(b) * p.geom.max_blocks + (tc >> 4)];
        phys = min(max(phys, 0), p.geom.num_pages - 1);
        row = (static_cast<int64_t>(phys) * p.geom.kvh + kvh) * kPageSize + (tc & (kPageSize - 1));
      } else {
        row = (static_cast<int64_t>(b) * p.geom.kvh + kvh) * p.geom.max_len + tc;
      }
      rowu[u] = row;
      kb[u] = zero_if_off(*reinterpret_cast<const uint4*>(p.k_codes + row * D + subc * 16));
      vb[u] = zero_if_off(*reinterpret_cast<const uint4*>(p.v_codes + row * D + subc * 16));
      ks[u] = FP8 || CH ? 1.0f : load_scale(p.k_scales, row * p.groups + grp, p.scale_bf16 != 0);
      vs[u] = FP8 || CH ? 1.0f : load_scale(p.v_scales, row * p.groups + grp, p.scale_bf16 != 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t kw[4] = {kb[u].x, kb[u].y, kb[u].z, kb[u].w};
      const uint32_t vw[4] = {vb[u].x, vb[u].y, vb[u].z, vb[u].w};
      float kscl[CH ? 16 : 1], vscl[CH ? 16 : 1];  // this lane's 16 channel scales of the token's block
      if constexpr (CH) {
        const int64_t sidx = (rowu[u] / kBlockRows) * D + subc * 16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 a = *reinterpret_cast<const float4*>(p.k_scales + sidx + 4 * i);
          const float4 c = *reinterpret_cast<const float4*>(p.v_scales + sidx + 4 * i);
          kscl[4 * i] = a.x; kscl[4 * i + 1] = a.y; kscl[4 * i + 2] = a.z; kscl[4 * i + 3] = a.w;
          vscl[4 * i] = c.x; vscl[4 * i + 1] = c.y; vscl[4 * i + 2] = c.z; vscl[4 * i + 3] = c.w;
        }
      }
      float part[HPW];
#pragma unroll
      for (int j = 0; j < HPW; ++j) part[j] = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float c = FP8 ? fp8_decode<E5>((kw[i] >> (8 * e)) & 0xffu) : byte_f32(kw[i], e);
          if constexpr (CH) c = fmaf(c, kscl[4 * i + e], -128.0f * kscl[4 * i + e]);  // fl32((c - 128) s)
#pragma unroll
          for (int j = 0; j < HPW; ++j) part[j] = fmaf(q[j][4 * i + e], c, part[j]);
        }
      float cv[16];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          cv[4 * i + e] = FP8 ? fp8_decode<E5>((vw[i] >> (8 * e)) & 0xffu) : byte_f32(vw[i], e);
          if constexpr (CH) cv[4 * i + e] = fmaf(cv[4 * i + e], vscl[4 * i + e], -128.0f * vscl[4 * i + e]);
        }
#pragma unroll
      for (int j = 0; j < HPW; ++j) {
        float sc = FP8 || CH ? part[j] : (part[j] - 128.0f * qsum[j]) * ks[u];
        sc = group_sum<LPT>(sc) * p.scale_log2;
        const float sj = ok[u] ? sc : -INFINITY;
        if (sj > m[j] + kLazy) {
          const float alpha = exp2f(m[j] - sj);
          l[j] *= alpha;
          ws[j] *= alpha;
#pragma unroll
          for (int e = 0; e < 16; ++e) o[j][e] *= alpha;
          m[j] = sj;
        }
        const float pj = ok[u] ? exp2f(sj - m[j]) : 0.0f;
        l[j] += pj;
        const float w = ok[u] ? pj * vs[u] : 0.0f;
        ws[j] += w;
#pragma unroll
        for (int e = 0; e < 16; ++e) o[j][e] = fmaf(w, cv[e], o[j][e]);
      }
    }
  }

  // ring rows (bf16 values, no scale and no offset): one token per lane slot
  // and pass, the same online softmax
  if (p.rwin > 0) {
    const int64_t ring0 = (static_cast<int64_t>(b) * p.geom.kvh + kvh) * p.rcap;
    for (int tb = max(t_begin, L8); tb < t_end; tb += TPP) {
      const int t = tb + wave * TPW + slot;
      const bool okr = t < t_end;
      const int64_t slot_row = ring0 + min(t, t_end - 1) % p.rcap;
      const uint4* kr = reinterpret_cast<const uint4*>(p.rk + slot_row * D + subc * 16);
      const uint4* vr = reinterpret_cast<const uint4*>(p.rv + slot_row * D + subc * 16);
      float kx[16], vx[16];
      bf16x8_to_f32(zero_if_off(kr[0]), &kx[0]);
      bf16x8_to_f32(zero_if_off(kr[1]), &kx[8]);
      bf16x8_to_f32(zero_if_off(vr[0]), &vx[0]);
      bf16x8_to_f32(zero_if_off(vr[1]), &vx[8]);
#pragma unroll
      for (int j = 0; j < HPW; ++j) {
        float part = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) part = fmaf(q[j][e], kx[e], part);
        const float sc = group_sum<LPT>(part) * p.scale_log2;
        const float sj = okr ? sc : -INFINITY;
        if (sj > m[j] + kLazy) {
          const float alpha = exp2f(m[j] - sj);
          l[j] *= alpha;
          ws[j] *= alpha;
#pragma unroll
          for (int e = 0; e < 16; ++e) o[j][e] *= alpha;
          m[j] = sj;
        }
        const float pj = okr ? exp2f(sj - m[j]) : 0.0f;
        l[j] += pj;
#pragma unroll
        for (int e = 0; e < 16; ++e) o[j][e] = fmaf(pj, vx[e], o[j][e]);
      }
    }
  }

#pragma unroll
  for (int j = 0; j < HPW; ++j) {
#pragma unroll
    for (int e = 0; e < 16; ++e) o[j][e] = FP8 || CH ? o[j][e] : fmaf(-128.0f, ws[j], o[j][e]);
    float M = m[j];
    for (int off = LPT; off < kWave; off <<= 1) M = fmaxf(M, __shfl_xor(M, off, kWave));
    const float f = (m[j] == -INFINITY) ? 0.0f : exp2f(m[j] - M);
    l[j] *= f;
#pragma unroll
    for (int e = 0; e < 16; ++e) o[j][e] *= f;
    for (int off = LPT; off < kWave; off <<= 1) {
      l[j] += __shfl_xor(l[j], off, kWave);
#pragma unroll
      for (int e = 0; e < 16; ++e) o[j][e] += __shfl_xor(o[j][e], off, kWave);
    }
    m[j] = M;
  }
  if (slot == 0 && sub_ok) {
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sm_o[wave][j][sub * 16 + e] = o[j][e];
      if (sub == 0) {
        sm_m[wave][j] = m[j];
        sm_l[wave][j] = l[j];
      }
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < HPW * D; idx += kThreads) {
    const int j = idx / D;
    const int d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][j]);
    float acc = 0.0f, lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = sm_m[w][j] == -INFINITY ? 0.0f : exp2f(sm_m[w][j] - M);
      acc = fmaf(sm_o[w][j][d], f, acc);
      lsum = fmaf(sm_l[w][j], f, lsum);
    }
    const int64_t pidx = (static_cast<int64_t>(v) * H + h0 + j) * p.num_splits + split;
    p.part_o[pidx * D + d] = acc;
    if (d == 0) {
      p.part_ml[pidx * 2] = M;
      p.part_ml[pidx * 2 + 1] = lsum;
    }
  }
}

// Every scale mode and heads-per-workgroup count of the generic kernel at
// head dim D.
template <int D>
void launch_generic_all(int hpw, int sm, bool paged, const DecodeParams& p, dim3 grid, hipStream_t st) {
  auto go = [&](auto hc, auto smc) {
    constexpr int HPW = decltype(hc)::value;
    constexpr int SM = decltype(smc)::value;
    if (paged) hipLaunchKernelGGL((decode_generic_kernel<D, HPW, SM, true>), grid, dim3(kThreads), 0, st, p);
    else hipLaunchKernelGGL((decode_generic_kernel<D, HPW, SM, false>), grid, dim3(kThreads), 0, st, p);
  };
  auto by_sm = [&](auto hc) {
    switch (sm) {
      case kSmGroup32: go(hc, std::integral_constant<int, kSmGroup32>{}); break;
      case kSmTokenBf16: go(hc, std::integral_constant<int, kSmTokenBf16>{}); break;
      case kSmFp8E4M3: go(hc, std::integral_constant<int, kSmFp8E4M3>{}); break;
      case kSmFp8E5M2: go(hc, std::integral_constant<int, kSmFp8E5M2>{}); break;
      case kSmBlockChannel: go(hc, std::integral_constant<int, kSmBlockChannel>{}); break;
      default: go(hc, std::integral_constant<int, kSmToken>{}); break;
    }
  };
  if (hpw == 4) by_sm(std::integral_constant<int, 4>{});
  else if (hpw == 2) by_sm(std::integral_constant<int, 2>{});
  else by_sm(std::integral_constant<int, 1>{});
}

}  // namespace

// The generic kernel at head dims 96, 160, 192 and 224 (kvq_decode_wide.hip).
void launch_generic_wide(int head_dim, int hpw, int sm, bool paged, const DecodeParams& p, dim3 grid,
                         hipStream_t st);

}  // namespace kvq
