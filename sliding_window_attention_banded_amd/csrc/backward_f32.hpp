// Backward pass for fp32 plans, written from the definition: for a non-global
// row i with key set A(i) = band(i) plus the global columns outside it, and
// for a global row g with every key (left of g when causal) of Qg, Kg, Vg
// (Longformer summary page, section 3-1, and section 7 for the causal mask):
//   P_ij = exp(s q_i.k_j - LSE_i),  D_i = dO_i . O_i,
//   dS_ij = P_ij (dO_i.v_j - D_i),
//   dq_i = s sum_j dS_ij k_j,  dk_j = s sum_i dS_ij q_i,  dv_j = sum_i P_ij dO_i.
// A correctness path for fp32 models: one wavefront per row (dq, dqg) or per
// key position (dk, dv, dkg, dvg), lane e holding feature e, dot products by
// cross-lane sums, fp32 throughout, every sum in a fixed order.
#pragma once

#include "backward.hpp"

namespace swattn {

DEV float wave_sum64(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Index of position i in the item's sorted set, or -1.
DEV int set_index(const GSet& gs, int i) {
  int lo = 0, hi = gs.n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (gs.idx[mid] < i) lo = mid + 1;
    else hi = mid;
  }
  return lo < gs.n && gs.idx[lo] == i ? lo : -1;
}

// Key j lies in row i's band: same residue class, i - half*dil <= j <= i + right*dil.
DEV bool in_band(int i, int j, const HeadGeom& hg) {
  const int dl = j - i;
  return dl % hg.dil == 0 && dl >= -hg.half * hg.dil && dl <= hg.right * hg.dil;
}

// D_i for every row: 16 lanes per row, four features each.
__global__ __launch_bounds__(256) void bwd_f32_prep(BwdParams p, long rows) {
  const long t = (long)blockIdx.x * 256 + threadIdx.x;
  const long row = t >> 4;
  const int part = threadIdx.x & 15;
  float acc = 0.f;
  if (row < rows) {
    const f32x4 a = reinterpret_cast<const f32x4*>(static_cast<const float*>(p.o) + row * HD)[part];
    const f32x4 b = reinterpret_cast<const f32x4*>(static_cast<const float*>(p.dout) + row * HD)[part];
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_fmaf(a[e], b[e], acc);
  }
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if (row < rows && part == 0) p.dd[row] = acc;
}

// One term of a row's or a key's gradient: the pair (row vectors qr, dor
// with LSE l and D dd; key vectors kr, vr) gives P and dS.
struct PairTerm { float p, ds; };
DEV PairTerm pair_term(float qe, float doe, float ke, float ve, float l, float dd, float scale) {
  const float s = wave_sum64(qe * ke);
  const float dp = wave_sum64(doe * ve);
  const float pr = expf(__builtin_fmaf(s, scale, -l));
  return PairTerm{pr, pr * (dp - dd)};
}

// dq (rows outside G) and dqg (rows of G): one wavefront per (b*h, row).
__global__ __launch_bounds__(256) void bwd_f32_rows(BwdParams p, long rows) {
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // wave-uniform
  const int e = threadIdx.x & 63;
  const long bh = row / p.n;
  const int i = (int)(row - bh * p.n);
  const HeadGeom hg = p.heads[bh % p.H];
  const GSet gs = batch_gset(p.gidx, p.goff, p.ng, (int)(bh / p.H));
  const long base = bh * (long)p.n * HD;
  const float* Q = static_cast<const float*>(p.q) + base;
  const float* K = static_cast<const float*>(p.k) + base;
  const float* V = static_cast<const float*>(p.v) + base;
  const float l = p.lse[row], dd = p.dd[row];
  const float doe = static_cast<const float*>(p.dout)[base + (long)i * HD + e];
  float acc = 0.f;
  if (gs.n > 0 && set_index(gs, i) >= 0) {
    // a global row: every key of Kg, Vg (left of it when causal)
    const float* KG = static_cast<const float*>(p.kg) + base;
    const float* VG = static_cast<const float*>(p.vg) + base;
    const float qe = static_cast<const float*>(p.qg)[base + (long)i * HD + e];
    const int jend = p.causal ? i + 1 : p.n;
    for (int j = 0; j < jend; ++j) {
      const float ke = KG[(long)j * HD + e];
      const PairTerm t = pair_term(qe, doe, ke, VG[(long)j * HD + e], l, dd, p.scale);
      acc = __builtin_fmaf(t.ds, ke, acc);
    }
    static_cast<float*>(p.dqg)[base + (long)i * HD + e] = acc * p.scale;
    static_cast<float*>(p.dq)[base + (long)i * HD + e] = 0.f;
    return;
  }
  const float qe = Q[(long)i * HD + e];
  // the band, in residue steps from -half to +right
  for (int t = -hg.half; t <= hg.right; ++t) {
    const long j = (long)i + (long)t * hg.dil;
    if (j < 0 || j >= p.n) continue;
    const float ke = K[j * HD + e];
    const PairTerm pt = pair_term(qe, doe, ke, V[j * HD + e], l, dd, p.scale);
    acc = __builtin_fmaf(pt.ds, ke, acc);
  }
  // the global columns outside the band (left of the row when causal)
  for (int a = 0; a < gs.n; ++a) {
    const int g = gs.idx[a];
    if (in_band(i, g, hg) || (p.causal && g > i)) continue;
    const float ke = K[(long)g * HD + e];
    const PairTerm pt = pair_term(qe, doe, ke, V[(long)g * HD + e], l, dd, p.scale);
    acc = __builtin_fmaf(pt.ds, ke, acc);
  }
  static_cast<float*>(p.dq)[base + (long)i * HD + e] = acc * p.scale;
  if (p.dqg) static_cast<float*>(p.dqg)[base + (long)i * HD + e] = 0.f;
}

// dk, dv (from the rows outside G whose key set holds j) and dkg, dvg (from
// the rows of G): one wavefront per (b*h, key position).
__global__ __launch_bounds__(256) void bwd_f32_keys(BwdParams p, long rows) {
  const long key = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (key >= rows) return;  // wave-uniform
  const int e = threadIdx.x & 63;
  const long bh = key / p.n;
  const int j = (int)(key - bh * p.n);
  const HeadGeom hg = p.heads[bh % p.H];
  const GSet gs = batch_gset(p.gidx, p.goff, p.ng, (int)(bh / p.H));
  const long base = bh * (long)p.n * HD;
  const long srow = bh * (long)p.n;  // this slice's first row of lse and D
  const float* Q = static_cast<const float*>(p.q) + base;
  const float* dO = static_cast<const float*>(p.dout) + base;
  const float ke = static_cast<const float*>(p.k)[base + (long)j * HD + e];
  const float ve = static_cast<const float*>(p.v)[base + (long)j * HD + e];
  float dk = 0.f, dv = 0.f;
  auto add_row = [&](int i) {
    const float qe = Q[(long)i * HD + e], doe = dO[(long)i * HD + e];
    const PairTerm t = pair_term(qe, doe, ke, ve, p.lse[srow + i], p.dd[srow + i], p.scale);
    dk = __builtin_fmaf(t.ds, qe, dk);
    dv = __builtin_fmaf(t.p, doe, dv);
  };
  // rows whose band holds j: i = j + u*dil, u from -right to +half
  for (int u = -hg.right; u <= hg.half; ++u) {
    const long i = (long)j + (long)u * hg.dil;
    if (i < 0 || i >= p.n) continue;
    if (gs.n > 0 && set_index(gs, (int)i) >= 0) continue;  // rows of G use Kg, Vg
    add_row((int)i);
  }
  if (gs.n > 0 && set_index(gs, j) >= 0) {
    // a global column: every other row outside G (right of j when causal)
    for (int i = p.causal ? j : 0; i < p.n; ++i) {
      if (in_band(i, j, hg) || set_index(gs, i) >= 0) continue;
      add_row(i);
    }
  }
  static_cast<float*>(p.dk)[base + (long)j * HD + e] = dk * p.scale;
  static_cast<float*>(p.dv)[base + (long)j * HD + e] = dv;
  if (!p.dkg) return;
  // Kg, Vg: the rows of G, left of position j excluded when causal
  const float kge = static_cast<const float*>(p.kg)[base + (long)j * HD + e];
  const float vge = static_cast<const float*>(p.vg)[base + (long)j * HD + e];
  float dkg = 0.f, dvg = 0.f;
  for (int a = 0; a < gs.n; ++a) {
    const int g = gs.idx[a];
    if (p.causal && j > g) continue;
    const float qe = static_cast<const float*>(p.qg)[base + (long)g * HD + e], doe = dO[(long)g * HD + e];
    const PairTerm t = pair_term(qe, doe, kge, vge, p.lse[srow + g], p.dd[srow + g], p.scale);
    dkg = __builtin_fmaf(t.ds, qe, dkg);
    dvg = __builtin_fmaf(t.p, doe, dvg);
  }
  static_cast<float*>(p.dkg)[base + (long)j * HD + e] = dkg * p.scale;
  static_cast<float*>(p.dvg)[base + (long)j * HD + e] = dvg;
}

}  // namespace swattn
