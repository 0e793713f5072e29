// Projection prologue: the linear projections that turn a layer's input into
// the attention's Q, K, V and, when global tokens are used, the separate
// Qg, Kg, Vg (Longformer summary page, section 3-1, "Linear Projections for
// Global Attention").
//
// For x [M = B*n, D] and a weight W [N = P*H*64, D] (one output feature per
// row, as a linear layer stores it) the kernel forms C^T = W x^T on the
// matrix cores and writes each 64-feature block of C (projection p, head h)
// straight into out[p][b][h][i][0..63], the layout the attention reads, with
// an optional bias added in fp32 before the bf16 rounding.
//
// Workgroup tile: 256 tokens x 256 features, 8 waves as 2 x 4 (one workgroup
// per CU), 256 tokens x 128 features, 4 waves as 2 x 2 (two per CU), or 128
// tokens x 128 features, 4 waves as 2 x 2 (three per CU); each wave 128 (64)
// tokens x 64 features = 4 (2) x 2 MFMA 32x32x16 tiles (PjCfg). Both operands are read k-contiguous (W rows and x rows), 32 input
// features per stage, through a 3-stage LDS ring filled by direct
// global->LDS loads, so that one wave's ring fill and stores run under the
// other waves' MFMAs.
#pragma once

#include "kernels.hpp"

namespace swattn {

constexpr int PJ_TN = 128;                                 // features per tile when choosing the shape
constexpr int PJ_TK = 32;                                  // input features per stage
constexpr int PJ_ROWB = PJ_TK * 2;                         // bytes per staged row (bf16)
constexpr int PJ_RPB = 1024 / PJ_ROWB;                     // rows per 1-KB load
constexpr int PJ_GROUP = 4;                                // token tiles swept together

// Workgroup shapes: TG 32-token groups per wave, so 2 * 32 * TG tokens per
// workgroup, and WN waves along 64 * WN output features. TG = 4, WN = 4: 256
// tokens x 256 features, a 96 KB ring (128 KB of LDS with the staged output
// tiles), one workgroup per CU: the W tile serves twice the tokens and the x
// tile twice the features of the 4-wave shape, so fewer staged bytes per MFMA
// (the encoder projection: 74 us against 78 us with 256 x 128 tiles of four
// waves, two per CU, and 88 us with TG = 2), when the problem still has two
// rounds of such workgroups; otherwise TG = 4, WN = 2, two per CU. TG = 2,
// WN = 2: 128 tokens x 128 features, a 48 KB ring, three per CU, for problems
// whose 256-token tiles cannot give every CU two workgroups (1024 tokens:
// 9.4 us against 13.9 us).
template <int TG, int WN = 2>
struct PjCfg {
  static constexpr int WT = 32 * TG;                       // tokens per wave
  static constexpr int TM = 2 * WT;                        // tokens per workgroup
  static constexpr int TN = 64 * WN;                       // output features per workgroup
  static constexpr int NW = 2 * WN;                        // waves: 2 along tokens, WN along features
  static constexpr int A_BYTES = TN * PJ_ROWB;             // W tile
  static constexpr int A_NI = A_BYTES / 1024;              // the first A_NI loads fill the W tile
  static constexpr int STAGE = A_BYTES + TM * PJ_ROWB;     // W + x tile per stage
  static constexpr int NI = STAGE / 1024;                  // 1-KB loads per stage
  static constexpr int PW = NI / NW;                       // loads per wave
  static constexpr int RING = 3 * STAGE;
  static constexpr int LDS = RING > NW * WT * 128 ? RING : NW * WT * 128;  // ring, then the staged tiles
  static_assert(NI % NW == 0, "loads split evenly over the waves");
};

struct ProjParams {
  const __bf16* x;     // [M][D]
  const __bf16* w;     // [N][D]
  const __bf16* bias;  // [N] or NULL
  __bf16* out;         // [P][B][H][n][64]
  int M;               // B * n
  int N;               // P * H * 64
  int D;               // multiple of 32
  int n;
  int B;
  int H;
  int tg;              // workgroup shape (PjCfg)
  int ntm;             // ceil(M / (64 * tg))
  int feat_base;       // first output feature of this launch
  int ntn;             // ceil(N / 128)
  int nblocks;         // ntm * ntn
};

// 16-byte chunk c of a 64-byte staged row sits at c ^ ((row >> 2) & 3): the
// 16 rows that 16 lanes read at one chunk then cover all 64 banks.
DEV int pj_phys(int row, int ch) { return ch ^ ((row >> 2) & 3); }
DEV int pj_off(int row, int ch) { return row * PJ_ROWB + (pj_phys(row, ch) << 4); }

// 16 bytes of an output row, non-temporal: the rows are written whole (eight
// lanes per 128-byte row) and stream out past L2 instead of staying dirty
// there until the kernel's end.
DEV void store_row16(__bf16* dst, const uint4& v) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(dst));
}

// Block -> (token tile, feature tile). xcd_remap gives each XCD a contiguous
// range of the order; the order runs over groups of PJ_GROUP token tiles and,
// within a group, feature-tile-major, so the blocks an XCD runs together
// share their few x tiles in L2 and each W tile is fetched once per group.
DEV void pj_tile(int bid, const ProjParams& p, int& tm, int& tn) {
  const int idx = xcd_remap(bid, p.nblocks);
  const int per = PJ_GROUP * p.ntn;
  const int grp = idx / per, r = idx - grp * per;
  const int gm = min(PJ_GROUP, p.ntm - grp * PJ_GROUP);
  tn = r / gm;
  tm = grp * PJ_GROUP + (r - tn * gm);
}

inline int proj_choose_tg(long M, long N, int cus) {
  const long big_tiles = (M + 255) / 256 * ((N + PJ_TN - 1) / PJ_TN);
  return big_tiles < 2L * cus ? 2 : 4;
}


template <int TG, int WN = 2>
__global__ __launch_bounds__(128 * WN, WN == 4 ? (TG == 4 ? 1 : 2) : (TG == 4 ? 2 : 3)) void proj_gemm(ProjParams p) {
  using C = PjCfg<TG, WN>;
  __shared__ __attribute__((aligned(1024))) char lds[C::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int tm, tn;
  pj_tile(blockIdx.x, p, tm, tn);
  const int tok0 = tm * C::TM, feat0 = p.feat_base + tn * C::TN;
  const unsigned lds0 = (unsigned)(uintptr_t)(lds_void*)lds;
  const unsigned rowbytes = (unsigned)p.D * 2u;

  // Load lane offsets: load I of a stage fills LDS rows 16*(I mod 8) .. +15
  // of the W tile (I < 8) or of the x tile; lane L writes the 16-byte slot
  // L of the 1-KB block, which holds logical chunk pj_phys(row, L % 4).
  unsigned doff[C::PW];
#pragma unroll
  for (int i = 0; i < C::PW; ++i) {
    const int I = wave * C::PW + i;
    const bool is_w = I < C::A_NI;
    const int row = (is_w ? I : I - C::A_NI) * PJ_RPB + (lane >> 2);
    const int grow = is_w ? min(feat0 + row, p.N - 1) : min(tok0 + row, p.M - 1);
    doff[i] = (unsigned)grow * rowbytes + ((unsigned)pj_phys(row, lane & 3) << 4);
  }
  auto issue = [&](int step, int stage) {
    const char* wb = reinterpret_cast<const char*>(p.w) + (size_t)step * PJ_ROWB;
    const char* xb = reinterpret_cast<const char*>(p.x) + (size_t)step * PJ_ROWB;
#pragma unroll
    for (int i = 0; i < C::PW; ++i) {
      const int I = wave * C::PW + i;
      dma16_saddr(I < C::A_NI ? wb : xb, doff[i],
                  lds0 + (unsigned)(stage * C::STAGE + I * 1024));
    }
  };

  // Fragment reads: lane l takes row l % 32 of a 32-row group, chunk
  // 2*ks + l/32 (input features 16*ks + 8*(l/32) .. +7); the swizzle reads
  // row bits 2..3 only, so the group enters as a plain offset.
  int roff[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) roff[ks] = pj_off(lane & 31, 2 * ks + (lane >> 5));
  const int wm = wave / WN, wn = wave % WN;
  const int a_off = wn * 64 * PJ_ROWB;                // this wave's 64 W rows
  const int b_off = C::A_BYTES + wm * C::WT * PJ_ROWB;  // this wave's x rows

  // This wave's 64 output features are one (projection, head) block; its
  // bias is read before the main loop so that the load's latency is hidden.
  const int ph = (feat0 >> 6) + wn;
  const bool ph_ok = ph * 64 < p.N;
  const int g = lane >> 5;
  bf16x4 bq[2][4];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int jq = 0; jq < 4; ++jq) {
      bq[f][jq] = bf16x4{};
      if (p.bias && ph_ok)
        bq[f][jq] = *reinterpret_cast<const bf16x4*>(p.bias + ph * 64 + f * 32 + 8 * jq + 4 * g);
    }

  f32x16 acc[2][TG];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int t = 0; t < TG; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[f][t][r] = 0.f;

  auto read_frags = [&](const char* sb, int ks, bf16x8 (&a)[2], bf16x8 (&b)[TG]) {
#pragma unroll
    for (int f = 0; f < 2; ++f)
      a[f] = *reinterpret_cast<const bf16x8*>(sb + a_off + f * 32 * PJ_ROWB + roff[ks]);
#pragma unroll
    for (int t = 0; t < TG; ++t)
      b[t] = *reinterpret_cast<const bf16x8*>(sb + b_off + t * 32 * PJ_ROWB + roff[ks]);
  };
  // MFMAs k0 .. k1-1 of one 16-feature step, k = TG * (feature group) + token group
  auto mma = [&](const bf16x8 (&a)[2], const bf16x8 (&b)[TG], int k0, int k1) {
#pragma unroll
    for (int k = 0; k < 2 * TG; ++k)
      if (k >= k0 && k < k1) acc[k / TG][k % TG] = mfma_bf16(a[k / TG], b[k % TG], acc[k / TG][k % TG]);
  };

  // Ring: stage s % 3 holds input features 32s .. 32s+31. Per stage: the
  // second 16-feature step's fragments are read under the first step's
  // MFMAs; the barrier that hands over the next stage and the loads that
  // refill this one go between the halves of the second step's MFMAs, and
  // the next stage's first fragments are read under its second half. The
  // last stage is peeled off so that the loop body has one path.
  const int nk = p.D / PJ_TK;
  issue(0, 0);
  if (nk > 1) issue(1, 1);
  if (nk > 1) wait_vmcnt<C::PW>();
  else wait_vmcnt<0>();
  wg_barrier();  // stage 0 has landed for every wave
  if (nk > 2) issue(2, 2);
  bf16x8 a0[2], b0[TG], a1[2], b1[TG];
  read_frags(lds, 0, a0, b0);
  int stage = 0;
  for (int s = 0; s + 1 < nk; ++s) {
    const char* sb = lds + stage * C::STAGE;
    const int nstage = stage == 2 ? 0 : stage + 1;
    read_frags(sb, 1, a1, b1);
    mma(a0, b0, 0, 2 * TG);
    if (s + 2 < nk) wait_vmcnt<C::PW>();
    else wait_vmcnt<0>();
    wait_lgkm0();  // this wave's reads of stage s have returned
    wg_barrier();  // stage s+1 has landed for every wave; stage s is consumed
    mma(a1, b1, 0, TG);
    if (s + 3 < nk) issue(s + 3, stage);
    read_frags(lds + nstage * C::STAGE, 0, a0, b0);
    mma(a1, b1, TG, 2 * TG);
    stage = nstage;
  }
  read_frags(lds + stage * C::STAGE, 1, a1, b1);
  mma(a0, b0, 0, 2 * TG);
  mma(a1, b1, 0, 2 * TG);

  // Epilogue. Lane l holds token column l % 32 of each 32-token group and,
  // in register j, feature 8*(j/4) + 4*(l/32) + j%4 of each 32-feature group.
  // Each wave stages its WT x 64 tile (bias added, rounded to bf16) in its
  // own WT * 128 bytes of the ring as [token][64 features], 8-byte unit u of row r at
  // u ^ ((r >> 1) & 15) (conflict-free for both access patterns), then
  // writes whole 128-byte token rows: 8 rows per store instruction.
  wait_lgkm0();
  wg_barrier();  // every wave is done with the ring
  if (!ph_ok) return;
  char* st = lds + wave * (C::WT * 128);
#pragma unroll
  for (int t = 0; t < TG; ++t) {
    const int row = t * 32 + (lane & 31);
    const int k = (row >> 1) & 15;
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        bf16x4 o4;
#pragma unroll
        for (int u = 0; u < 4; ++u) o4[u] = (__bf16)(acc[f][t][4 * jq + u] + (float)bq[f][jq][u]);
        const int unit = (f * 8 + 2 * jq + g) ^ k;
        *reinterpret_cast<bf16x4*>(st + row * 128 + unit * 8) = o4;
      }
  }
  wait_lgkm0();  // the wave reads back what its other lanes wrote
  const int proj = ph / p.H, h = ph - proj * p.H;
  const int T = tok0 + wm * C::WT;  // this wave's first token
  __bf16* obase = p.out + ((size_t)proj * p.B * p.H + h) * (size_t)p.n * 64;
  const size_t item_stride = (size_t)p.H * p.n * 64;
  const int item0 = T / p.n, pos0 = T - item0 * p.n;
  const bool one_item = pos0 + C::WT <= p.n;  // wave-uniform
  if (one_item && T + C::WT <= p.M) {
    // every row exists and the wave's rows are consecutive in out: read the
    // whole tile back first, then store it without per-lane conditions
    __bf16* orow = obase + item0 * item_stride + (size_t)pos0 * 64;
    uint4 v[C::WT / 8];
#pragma unroll
    for (int it = 0; it < C::WT / 8; ++it) {
      const int row = it * 8 + (lane >> 3), c = lane & 7;
      const int k = (row >> 1) & 15;
      v[it] = *reinterpret_cast<const uint4*>(st + row * 128 + ((c ^ (k >> 1)) << 4));
      if (k & 1) v[it] = uint4{v[it].z, v[it].w, v[it].x, v[it].y};
    }
#pragma unroll
    for (int it = 0; it < C::WT / 8; ++it)
      store_row16(orow + (size_t)(it * 8 + (lane >> 3)) * 64 + (lane & 7) * 8, v[it]);
    return;
  }
#pragma unroll
  for (int it = 0; it < C::WT / 8; ++it) {
    const int row = it * 8 + (lane >> 3), c = lane & 7;
    const int k = (row >> 1) & 15;
    uint4 v = *reinterpret_cast<const uint4*>(st + row * 128 + ((c ^ (k >> 1)) << 4));
    if (k & 1) v = uint4{v.z, v.w, v.x, v.y};
    const int tok = T + row;
    if (tok < p.M) {
      int b = item0, i = pos0 + row;
      if (!one_item) { b = tok / p.n; i = tok - b * p.n; }
      store_row16(obase + b * item_stride + (size_t)i * 64 + c * 8, v);
    }
  }
}

// ----------------------------------------------------------------------------
// fp32 projections: the same map and output layout with x, w, bias and out
// in fp32, for the fp32 attention path. On the vector ALUs (fp32 FMAs in
// input-feature order, so the result is a plain fp32 dot product): a
// workgroup computes 64 tokens x one 64-feature (projection, head) block,
// staging 16 input features of x and w at a time in LDS; each thread owns
// 4 tokens x 4 features.

struct ProjParamsF32 {
  const float* x;     // [M][D]
  const float* w;     // [N][D]
  const float* bias;  // [N] or NULL
  float* out;         // [P][B][H][n][64]
  int M, N, D, n, B, H;
  int nph;            // N / 64 feature blocks
};

__global__ __launch_bounds__(256) void proj_f32(ProjParamsF32 p) {
  constexpr int TT = 64, TK = 16;
  __shared__ float xs[TK][TT + 4];  // [input feature][token]
  __shared__ float ws[TK][TT + 4];  // [input feature][output feature]
  const int ph = blockIdx.x % p.nph, tm = blockIdx.x / p.nph;
  const int tok0 = tm * TT, f0 = ph * HD;
  const int tid = threadIdx.x, ti = tid >> 4, tj = tid & 15;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  for (int k0 = 0; k0 < p.D; k0 += TK) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = tid + 256 * u, row = idx >> 4, kk = idx & 15;
      const int tok = min(tok0 + row, p.M - 1);  // rows past M are computed, never stored
      xs[kk][row] = p.x[(long)tok * p.D + k0 + kk];
      ws[kk][row] = p.w[(long)(f0 + row) * p.D + k0 + kk];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = xs[kk][4 * ti + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = ws[kk][4 * tj + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  const int proj = ph / p.H, h = ph - proj * p.H;
  float bj[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) bj[j] = p.bias ? p.bias[f0 + 4 * tj + j] : 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tok = tok0 + 4 * ti + i;
    if (tok >= p.M) continue;
    const int b = tok / p.n, pos = tok - b * p.n;
    float* orow = p.out + ((((size_t)proj * p.B + b) * p.H + h) * p.n + pos) * HD;
    f32x4 v;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = acc[i][j] + bj[j];
    *reinterpret_cast<f32x4*>(orow + 4 * tj) = v;
  }
}

}  // namespace swattn
