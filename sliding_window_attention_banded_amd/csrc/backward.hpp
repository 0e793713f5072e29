// Device kernels of the backward pass (bf16), built from the forward's
// machinery (kernels.hpp): residue-class tiles, the direct-to-LDS ring, the
// 32-key unit and its MFMA layouts.
//
// For a cotangent dO of O and the forward's LSE, with P_ij = exp(s q_i.k_j -
// LSE_i) over the row's key set A(i) (Longformer summary page, section 3-1):
//   D_i   = dO_i . O_i                 (= sum_j P_ij dO_i.v_j)
//   dS_ij = P_ij (dO_i.v_j - D_i)
//   dq_i  = s sum_j dS_ij k_j,   dk_j = s sum_i dS_ij q_i,   dv_j = sum_i P_ij dO_i.
// Rows of G take their output from the global projections only, so the band
// passes treat them as absent: their log2-LSE is set to +inf (P = 0).
//
// Kernels:
//  * bwd_prep: D_i and the log2-domain LSE (+inf on rows of G), per row; the
//    same statistics of the global rows in a padded [BH][ngp] table.
//  * bwd_main, band query blocks: 128 query rows of one residue class, Q and
//    dO in registers, key tiles (K, V) through the ring, the global-column
//    tile first: dq = s dS K; and the zero rows of dqg off G.
//  * bwd_main, band key blocks: 128 keys of one residue class, K and V in
//    registers, query tiles (Q, dO, log2-LSE, D) through the ring: dk, dv.
//  * bwd_main, global-row query blocks: rows of G (Qg, dO) against a chunk of
//    Kg, Vg: a dQg partial per chunk.
//  * bwd_main, global-row key blocks: 128 positions of Kg, Vg against the
//    gathered rows of G: dKg, dVg.
//  * bwd_main, global-column key blocks: 32 keys of G (K, V) per wave
//    against a chunk of query positions: partial dK[G], dV[G] terms of the
//    rows whose band does not hold the key.
//  * bwd_gred: sums the partials into dqg and into rows G of dk and dv.
//
// Score tiles again come out transposed from the MFMA so that the
// probabilities (and dS) are already the B operand of the next product:
//  * query blocks: S^T = K Q^T and dP^T = V dO^T (lane = query), then
//    dQ^T += K^T dS^T with K^T read transposed from LDS;
//  * key blocks: T = Q K^T and dP = dO V^T (lane = key; Q, dO rows fed in
//    the permuted row order), then dV^T += dO^T P and dK^T += Q^T dS with
//    dO^T, Q^T read transposed from LDS.
#pragma once

#include "kernels.hpp"

namespace swattn {

// Per-head band geometry for the global-column blocks.
struct HeadGeom { int half, right, dil, pad; };

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* qg;
  const void* kg;
  const void* vg;
  const void* o;
  const void* dout;
  const float* lse;   // [BH][n], natural log (the forward's output)
  void* dq;
  void* dk;
  void* dv;
  void* dqg;
  void* dkg;
  void* dvg;
  float* lse2;        // [BH][n]: LSE * log2(e), +inf on rows of G
  float* dd;          // [BH][n]: D
  float* glse2;       // [BH][ngp]: LSE * log2(e) of the global rows (+inf padding)
  float* gdd;         // [BH][ngp]: D of the global rows (0 padding)
  float* part_dqg;    // [BH][ng][nsplit][64]: dQg partial per key chunk (unscaled)
  float* part_gkv;    // [BH][nchunk][ng32][128]: dK[G] (unscaled), dV[G] partial per query chunk
  const TileRec* tiles;
  const HeadGeom* heads;  // [H]
  int uni_half, uni_right, uni_dil, uni_nqb;
  const int* gidx;        // as in BandParams: one set, or per-item sets
  const int* goff;        // [B+1] or NULL
  int ng, ngp, ng32;      // ng: |G| or the largest per-item |G|
  int n, H;
  int causal;
  int nsplit, ksplit, nqb, ngroup;  // dQg blocks (as in the forward's global rows)
  int nchunk, gcol_qc;              // query chunks of the global-column blocks, their size
  int nkgb;                         // groups of 4 x 32 global keys
  // block counts of bwd_main: band query blocks (nq), band key blocks (nq),
  // dQg blocks, dKg/dVg blocks, global-column blocks
  int nq, n_gq, n_gkv, n_gcol;
  // 1: one global token per item; the global rows (dQg partials, dKg, dVg)
  // and the global columns are streamed on the vector ALUs (n_gkv = 0),
  // by the bwd_main<true> instantiation
  int gstream;
  float c2;           // scale * log2(e)
  float scale;
};

// Query positions per global-column block, and keys per dQg block. With at
// most 32 global tokens per item those blocks compute little and mostly wait
// on memory, so they are made fewer and longer (about a quarter of the
// sequence per global-column block, within [512, 4096], and at least 1024
// keys per dQg block), holding fewer workgroup slots; longer still and they
// become the critical path. Larger sets keep the finer split.
constexpr int GCOL_QC = 512;
constexpr int GCOL_QC_MAX = 4096;
constexpr int GQ_KEYS_SMALL_G = 1024;

// ----------------------------------------------------------------------------
// Row statistics: 4 lanes per row, 16 elements (two 16-byte loads) each.

__global__ __launch_bounds__(256) void bwd_prep(BwdParams p, long rows) {
  const long t = (long)blockIdx.x * 256 + threadIdx.x;
  const long row = t >> 2;
  const int part = threadIdx.x & 3;
  float acc = 0.f;
  if (row < rows) {
    const bf16x8* ap = reinterpret_cast<const bf16x8*>(reinterpret_cast<const __bf16*>(p.o) + row * HD + 16 * part);
    const bf16x8* bp = reinterpret_cast<const bf16x8*>(reinterpret_cast<const __bf16*>(p.dout) + row * HD + 16 * part);
    const bf16x8 a0 = ap[0], a1 = ap[1], b0 = bp[0], b1 = bp[1];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)a0[e], (float)b0[e], acc);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)a1[e], (float)b1[e], acc);
  }
  // sum the 4 lanes of the row (aligned groups of 4 within the wave)
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  const long rowc = row < rows ? row : rows - 1;
  const GSet gs = batch_gset(p.gidx, p.goff, p.ng, (int)(rowc / p.n / p.H));
  if (row < rows && part == 0) {
    const int i = (int)(row % p.n);
    // each set is sorted: binary search for i
    int lo = 0, hi = gs.n;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (gs.idx[mid] < i) lo = mid + 1;
      else hi = mid;
    }
    const bool isg = lo < gs.n && gs.idx[lo] == i;
    p.lse2[row] = isg ? __builtin_inff() : p.lse[row] * LOG2E;
    p.dd[row] = acc;
    if (isg) {
      const long bh = row / p.n;
      p.glse2[bh * p.ngp + lo] = p.lse[row] * LOG2E;
      p.gdd[bh * p.ngp + lo] = acc;
    }
  }
}

// ----------------------------------------------------------------------------
// Shared pieces.


// A pair of fp32 accumulators for a 64-wide row block of 32 lanes (the same
// layout as the forward's O^T accumulator).
struct Acc2 { f32x16 a[2]; };

DEV void acc2_zero(Acc2& x) {
#pragma unroll
  for (int i = 0; i < 16; ++i) { x.a[0][i] = 0.f; x.a[1][i] = 0.f; }
}

DEV void acc2_mma(Acc2& x, const VFrag& v, const PFrag& pf) {
#pragma unroll
  for (int sp = 0; sp < 2; ++sp)
#pragma unroll
    for (int dh = 0; dh < 2; ++dh) x.a[dh] = mfma_bf16(v.a[sp][dh], pf.b[sp], x.a[dh]);
}

// Row of 64 for this lane (lane l and l^32 hold alternate 4-element groups).
DEV void store_row(__bf16* row, const Acc2& x, float f, int g) {
#pragma unroll
  for (int dh = 0; dh < 2; ++dh)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      bf16x4 t;
#pragma unroll
      for (int e = 0; e < 4; ++e) t[e] = (__bf16)(x.a[dh][4 * a + e] * f);
      *reinterpret_cast<bf16x4*>(row + 32 * dh + 8 * a + 4 * g) = t;
    }
}

// Two f32x16 into the bf16 B-operand fragment (register j of the accumulator
// is element j%8 of step j/8, as for P in the forward).
DEV PFrag to_bfrag(const f32x16& x) {
  PFrag pf;
#pragma unroll
  for (int j = 0; j < 16; j += 2) {
    const bf16x2 t = __builtin_convertvector(f32x2{x[j], x[j + 1]}, bf16x2);
    pf.b[j >> 3][j & 7] = t[0];
    pf.b[j >> 3][(j & 7) + 1] = t[1];
  }
  return pf;
}

// ----------------------------------------------------------------------------
// Query blocks: dq.

struct DqWave {
  QFrag<__bf16> qf, dof;
  float lse2, dd;
  Acc2 dq;
};

// One 32-key unit of a K/V tile in LDS (K at kbuf, V at vbuf); `mask` is
// applied to the raw scores before the exponential. With SPLIT, dS enters
// its MFMA as a bf16 pair hi + lo (hi = bf16(dS), lo = bf16(dS - hi)), which
// keeps 16 significant bits: used for the global rows, whose dq sums the
// terms of every key and cancels the most.
template <bool SPLIT = false, class MaskFn>
DEV void dq_unit(DqWave& w, const char* kbuf, const char* vbuf, int kh, const LdsLanes& ll,
                 float c2, bool need_mask, MaskFn&& mask) {
  f32x16 s = score_from(load_kfrag(kbuf, kh, ll), w.qf);
  const f32x16 dp = score_from(load_kfrag(vbuf, kh, ll), w.dof);
  const VFrag kt = load_vfrag(kbuf, kh, ll);  // K^T, in flight during the VALU work
  if (need_mask) mask(s);
  f32x16 ds;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float pj = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j], c2, -w.lse2));
    ds[j] = pj * (dp[j] - w.dd);
  }
  const PFrag hi = to_bfrag(ds);
  acc2_mma(w.dq, kt, hi);
  if constexpr (SPLIT) {
    f32x16 lo;
#pragma unroll
    for (int j = 0; j < 16; ++j) lo[j] = ds[j] - (float)hi.b[j >> 3][j & 7];
    acc2_mma(w.dq, kt, to_bfrag(lo));
  }
}

// The ring for query blocks (K/V tiles, as in the forward).
template <int S, bool SPLIT = false, class Pol>
DEV void dq_ring_step(int tb, DqWave& w, const RingCtx& c, const Pol& pol, const DmaLanes<__bf16>& dl,
                      const char* st0, const char* st1, const char* st2) {
  constexpr int TILEB = KT * ElemTraits<__bf16>::ROWB;
  const char* cur = S == 0 ? st0 : (S == 1 ? st1 : st2);
  constexpr int SN = (S + 2) % 3;
  const unsigned nxt = SN == 0 ? c.a0 : (SN == 1 ? c.a1 : c.a2);
  wait_vmcnt<Dma<__bf16>::PER_WAVE>();
  wg_barrier();
  const int kn = c.kbeg + ring_tile(c, min(tb + 2, c.nband - 1)) * KT;
  if (kn + KT <= c.kend) dma_tile_fast<__bf16>(nxt, dl, c.kb, c.vb, kn, c.r, c.dil, c.wave);
  else dma_tile<__bf16>(nxt, c.kb, c.vb, kn, c.kend, c.r, c.dil, c.wave, c.lane);
  if (!c.live) return;
  const int k0 = c.kbeg + ring_tile(c, tb) * KT;
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
    const int ku = k0 + 32 * kh;
    if (!pol.active(ku)) continue;
    dq_unit<SPLIT>(w, cur, cur + TILEB, kh, c.ll, c.c2, !pol.interior(ku),
                   [&](f32x16& s) { pol.template mask<__bf16>(s, ku, c.g); });
  }
}

DEV void bwd_dq_block(const BwdParams& p, int tile, char* st0, char* st1, char* st2, int (*gmeta)[KT]) {
  constexpr int ROWB = ElemTraits<__bf16>::ROWB;
  constexpr int TILEB = KT * ROWB;
  const int tid = threadIdx.x;
  const int lane = tid & 63, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  BandParams bp{};  // the tile decode reads only these fields
  bp.tiles = p.tiles; bp.uni_half = p.uni_half; bp.uni_right = p.uni_right;
  bp.uni_dil = p.uni_dil; bp.uni_nqb = p.uni_nqb; bp.n = p.n;
  const TileRec td = decode_tile(bp, tile);
  const GSet gs = batch_gset(p.gidx, p.goff, p.ng, td.bh / p.H);
  const int* gix = gs.idx;
  const int ngb = gs.n;
  int gq[4] = {0, 0, 0, 0};
  int gm = 0;
  int gpos1 = 0;  // the global column when it is the only one
  if (ngb > 1) {
    gather_rows(gq, gix, 0, ngb, wave, lane);
    gm = gix[min(lane, ngb - 1)];
  } else if (ngb == 1) {
    gpos1 = gix[0];
  }
  const int bh = td.bh, r = td.r, q0 = td.q0, nr = td.nr;
  if (q0 >= nr) return;
  const int half = td.half, right = td.right, dil = td.dil;
  const long base = (long)bh * p.n * ROWB;
  const char* kb = reinterpret_cast<const char*>(p.k) + base;
  const char* vb = reinterpret_cast<const char*>(p.v) + base;
  const int kbeg = max(0, q0 - half);
  const int kend = min(nr, q0 + BM + right);
  const int nband = (kend - kbeg + KT - 1) / KT;
  const int qw0 = q0 + 32 * wave;
  const bool wave_live = qw0 < nr;
  const int qi = qw0 + (lane & 31);
  const bool row_ok = qi < nr;
  const int pos_q = r + min(qi, nr - 1) * dil;
  const int lim = p.causal ? pos_q : 0x7fffffff - 1;

  RingCtx c{(unsigned)(uintptr_t)(lds_void*)st0, (unsigned)(uintptr_t)(lds_void*)st1,
            (unsigned)(uintptr_t)(lds_void*)st2, kb, vb, kbeg, kend, nband, r, dil,
            wave, lane, g, wave_live, p.c2, {}};
  lds_lanes_init(c.ll, lane);
  // neighbouring blocks start on the key tile they share, as in the forward
  c.rot = band_rotation(q0, kbeg, nband, half, right);
  const BandPol pol{qi, qw0, half, right, nr, max(0, qw0 - half), min(nr - 1, qw0 + 31 + right)};

  DqWave w;
  acc2_zero(w.dq);
  const long roff = base + (long)pos_q * ROWB;
  if (ngb > 1) dma_gather(c.a2, kb, vb, gq, wave, lane);
  ring_start<__bf16>(c);
  load_q(w.qf, reinterpret_cast<const __bf16*>(reinterpret_cast<const char*>(p.q) + roff), g);
  load_q(w.dof, reinterpret_cast<const __bf16*>(reinterpret_cast<const char*>(p.dout) + roff), g);
  w.lse2 = p.lse2[(long)bh * p.n + pos_q];
  w.dd = p.dd[(long)bh * p.n + pos_q];
  if (ngb == 1) {
    // One global column: its term from registers, as the forward folds it
    // in. Score and dP are dot products over the row's two lanes; the dS
    // weight is rounded to bf16 like the units' B operand.
    QFrag<__bf16> kgf, vgf;
    bf16x4 kacc[2][4];
    const __bf16* krow = reinterpret_cast<const __bf16*>(kb + (long)gpos1 * ROWB);
    load_q(kgf, krow, g);
    load_q(vgf, reinterpret_cast<const __bf16*>(vb + (long)gpos1 * ROWB), g);
#pragma unroll
    for (int dh = 0; dh < 2; ++dh)
#pragma unroll
      for (int a = 0; a < 4; ++a) kacc[dh][a] = *reinterpret_cast<const bf16x4*>(krow + 32 * dh + 8 * a + 4 * g);
    wait_vmcnt<0>();
    if (wave_live) {
      float sp = 0.f, dpp = 0.f;
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          sp = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{w.qf.v[st][e], w.qf.v[st][e + 1]},
                                               bf16x2{kgf.v[st][e], kgf.v[st][e + 1]}, sp, false);
          dpp = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{w.dof.v[st][e], w.dof.v[st][e + 1]},
                                                bf16x2{vgf.v[st][e], vgf.v[st][e + 1]}, dpp, false);
        }
      const float sc = pair_sum(sp), dp = pair_sum(dpp);
      const int dr = gpos1 - r;
      const bool same = dr >= 0 && dr % dil == 0;
      const bool inband = same && dr / dil >= qi - half && dr / dil <= qi + right;
      const float pj = gpos1 <= lim && !inband ? __builtin_amdgcn_exp2f(__builtin_fmaf(sc, p.c2, -w.lse2)) : 0.f;
      const float ds = (float)(__bf16)(pj * (dp - w.dd));
#pragma unroll
      for (int dh = 0; dh < 2; ++dh)
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int e = 0; e < 4; ++e) w.dq.a[dh][4 * a + e] = __builtin_fmaf(ds, (float)kacc[dh][a][e], w.dq.a[dh][4 * a + e]);
    }
  } else if (ngb > 1) {
    if (tid < KT) gmeta_write(gmeta, gm, tid < ngb, r, dil, tid);
    wait_vmcnt<0>();
    __syncthreads();
    for (int t0 = 0;;) {
      if (wave_live) {
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          if (t0 + 32 * kh >= ngb) continue;
          dq_unit(w, st2, st2 + TILEB, kh, c.ll, p.c2, true, [&](f32x16& s) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              const int kk = 32 * kh + key_of_reg<__bf16>(j, g);
              const int kp = gmeta[0][kk], kr = gmeta[1][kk];
              const bool inband = kr >= qi - half && kr <= qi + right;
              if (!(kp <= lim) || inband) s[j] = -__builtin_inff();
            }
          });
        }
      }
      t0 += KT;
      if (t0 >= ngb) break;
      gather_rows(gq, gix, t0, ngb, wave, lane);
      gm = gix[min(t0 + lane, ngb - 1)];
      __syncthreads();
      dma_gather(c.a2, kb, vb, gq, wave, lane);
      if (tid < KT) gmeta_write(gmeta, gm, t0 + tid < ngb, r, dil, tid);
      wait_vmcnt<0>();
      __syncthreads();
    }
  } else {
    wait_vmcnt<0>();
  }

  DmaLanes<__bf16> dl;
  dma_lanes_init<__bf16>(dl, dil, lane);
  for (int tb = 0; tb < nband; tb += 3) {
    dq_ring_step<0>(tb, w, c, pol, dl, st0, st1, st2);
    if (tb + 1 < nband) dq_ring_step<1>(tb + 1, w, c, pol, dl, st0, st1, st2);
    if (tb + 2 < nband) dq_ring_step<2>(tb + 2, w, c, pol, dl, st0, st1, st2);
  }
  wait_vmcnt<0>();

  if (wave_live) {
    // whole-row stores through the stage of ring step nband (free: see the
    // forward's band blocks)
    const int sa = nband % 3;
    char* slot = (sa == 0 ? st0 : (sa == 1 ? st1 : st2)) + 4096 * wave;
    store_o_rows(slot, reinterpret_cast<char*>(p.dq) + base, w.dq.a, p.scale, lane, qw0, nr, r, dil);
    // dQg is zero off G (rows of G, log2-LSE +inf, come from bwd_gred): lane
    // i writes 16 bytes of row 8k + i/8, whose log2-LSE lane 8k + i/8 holds
    if (p.dqg) {
      typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int row = 8 * k + (lane >> 3);
        const float l2 = __shfl(w.lse2, row);
        if (qw0 + row < nr && l2 != __builtin_inff())
          __builtin_nontemporal_store(
              u32x4{0u, 0u, 0u, 0u},
              reinterpret_cast<u32x4*>(reinterpret_cast<char*>(p.dqg) + base +
                                       (long)(r + (qw0 + row) * dil) * ROWB + (lane & 7) * 16));
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Key blocks: dk, dv.
//
// A ring stage holds a tile of 64 query rows: Q (8 KB), dO (8 KB) and the
// rows' log2-LSE and D (256 B each, in the first 512 B of a 1 KB area that
// the four waves fill: waves 0 and 2 load the log2-LSE, waves 1 and 3 D, the
// latter pair into a second copy that nobody reads, so that every wave
// issues the same number of loads).

constexpr int QSTAGEB = 2 * KT * 128 + 1024;

struct DkvWave {
  QFrag<__bf16> kf, vf;  // this lane's key row of K and of V (B operands)
  Acc2 dk, dv;
};

DEV void dma_stats(unsigned stage, const float* lse2, const float* dd, int kb0, int kend, int r,
                   int dil, int wave, int lane) {
  const int kk = min(kb0 + lane, kend - 1);
  const float* src = ((wave & 1) ? dd : lse2) + (r + (long)kk * dil);
  dma4(src, stage + (unsigned)(2 * KT * 128 + 256 * wave));
}

// One 32-query unit (rows 32*kh.. of the tile at `stage`).
template <class MaskFn>
DEV void dkv_unit(DkvWave& w, const char* stage, int kh, const LdsLanes& ll, float c2, int g,
                  bool need_mask, MaskFn&& mask) {
  constexpr int TILEB = KT * 128;
  f32x16 t = score_from(load_kfrag(stage, kh, ll), w.kf);           // T[q][key]
  const f32x16 dp = score_from(load_kfrag(stage + TILEB, kh, ll), w.vf);  // dP[q][key]
  // register j holds query 16*(j/8) + 8g + j%8 of the unit
  const float* sl = reinterpret_cast<const float*>(stage + 2 * TILEB) + 32 * kh + 8 * g;
  const float* sd = reinterpret_cast<const float*>(stage + 2 * TILEB + 256) + 32 * kh + 8 * g;
  const f32x4 l0 = *reinterpret_cast<const f32x4*>(sl), l1 = *reinterpret_cast<const f32x4*>(sl + 4);
  const f32x4 l2 = *reinterpret_cast<const f32x4*>(sl + 16), l3 = *reinterpret_cast<const f32x4*>(sl + 20);
  const f32x4 d0 = *reinterpret_cast<const f32x4*>(sd), d1 = *reinterpret_cast<const f32x4*>(sd + 4);
  const f32x4 d2 = *reinterpret_cast<const f32x4*>(sd + 16), d3 = *reinterpret_cast<const f32x4*>(sd + 20);
  const VFrag dot = load_vfrag(stage + TILEB, kh, ll);  // dO^T
  const VFrag qt = load_vfrag(stage, kh, ll);           // Q^T
  if (need_mask) mask(t);
  f32x16 pj, ds;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int a = j >> 2, e = j & 3;
    const float l2j = a == 0 ? l0[e] : a == 1 ? l1[e] : a == 2 ? l2[e] : l3[e];
    const float ddj = a == 0 ? d0[e] : a == 1 ? d1[e] : a == 2 ? d2[e] : d3[e];
    pj[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(t[j], c2, -l2j));
    ds[j] = pj[j] * (dp[j] - ddj);
  }
  acc2_mma(w.dv, dot, to_bfrag(pj));
  acc2_mma(w.dk, qt, to_bfrag(ds));
}

template <int S, class Pol>
DEV void dkv_ring_step(int tb, DkvWave& w, const RingCtx& c, const Pol& pol, const DmaLanes<__bf16>& dl,
                       const float* lse2, const float* dd, const char* st0, const char* st1,
                       const char* st2) {
  const char* cur = S == 0 ? st0 : (S == 1 ? st1 : st2);
  constexpr int SN = (S + 2) % 3;
  const unsigned nxt = SN == 0 ? c.a0 : (SN == 1 ? c.a1 : c.a2);
  wait_vmcnt<Dma<__bf16>::PER_WAVE + 1>();
  wg_barrier();
  const int kn = c.kbeg + ring_tile(c, min(tb + 2, c.nband - 1)) * KT;
  if (kn + KT <= c.kend) dma_tile_fast<__bf16>(nxt, dl, c.kb, c.vb, kn, c.r, c.dil, c.wave);
  else dma_tile<__bf16>(nxt, c.kb, c.vb, kn, c.kend, c.r, c.dil, c.wave, c.lane);
  dma_stats(nxt, lse2, dd, kn, c.kend, c.r, c.dil, c.wave, c.lane);
  if (!c.live) return;
  const int k0 = c.kbeg + ring_tile(c, tb) * KT;
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
    const int ku = k0 + 32 * kh;
    if (!pol.active(ku)) continue;
    dkv_unit(w, cur, kh, c.ll, c.c2, c.g, !pol.interior(ku),
             [&](f32x16& s) { pol.template mask<__bf16>(s, ku, c.g); });
  }
}

DEV void bwd_dkv_block(const BwdParams& p, int tile, char* st0, char* st1, char* st2) {
  constexpr int ROWB = ElemTraits<__bf16>::ROWB;
  const int tid = threadIdx.x;
  const int lane = tid & 63, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  BandParams bp{};
  bp.tiles = p.tiles; bp.uni_half = p.uni_half; bp.uni_right = p.uni_right;
  bp.uni_dil = p.uni_dil; bp.uni_nqb = p.uni_nqb; bp.n = p.n;
  const TileRec td = decode_tile(bp, tile);
  const int bh = td.bh, r = td.r, k0 = td.q0, nr = td.nr;
  if (k0 >= nr) return;
  const int half = td.half, right = td.right, dil = td.dil;
  const long base = (long)bh * p.n * ROWB;
  // key j is seen by query i iff i - half <= j <= i + right, i.e. by the
  // queries j - right .. j + half: the band with its two sides exchanged
  const int qbeg = max(0, k0 - right);
  const int qend = min(nr, k0 + BM + half);
  const int nband = (qend - qbeg + KT - 1) / KT;
  const int kw0 = k0 + 32 * wave;
  const bool wave_live = kw0 < nr;
  const int kj = kw0 + (lane & 31);
  const bool key_ok = kj < nr;
  const int pos_k = r + min(kj, nr - 1) * dil;

  RingCtx c{(unsigned)(uintptr_t)(lds_void*)st0, (unsigned)(uintptr_t)(lds_void*)st1,
            (unsigned)(uintptr_t)(lds_void*)st2,
            reinterpret_cast<const char*>(p.q) + base, reinterpret_cast<const char*>(p.dout) + base,
            qbeg, qend, nband, r, dil, wave, lane, g, wave_live, p.c2, {}};
  lds_lanes_init(c.ll, lane);
  // neighbouring blocks start on the query tile they share
  c.rot = band_rotation(k0, qbeg, nband, right, half);
  const BandPol pol{kj, kw0, right, half, nr, max(0, kw0 - right), min(nr - 1, kw0 + 31 + half)};
  const float* lse2 = p.lse2 + (long)bh * p.n;
  const float* dd = p.dd + (long)bh * p.n;

  DkvWave w;
  acc2_zero(w.dk);
  acc2_zero(w.dv);
  const long roff = base + (long)pos_k * ROWB;
  const int q0t = qbeg + ring_tile(c, 0) * KT;
  dma_tile<__bf16>(c.a0, c.kb, c.vb, q0t, qend, r, dil, wave, lane);
  dma_stats(c.a0, lse2, dd, q0t, qend, r, dil, wave, lane);
  const int q1 = qbeg + ring_tile(c, min(1, nband - 1)) * KT;
  dma_tile<__bf16>(c.a1, c.kb, c.vb, q1, qend, r, dil, wave, lane);
  dma_stats(c.a1, lse2, dd, q1, qend, r, dil, wave, lane);
  load_q(w.kf, reinterpret_cast<const __bf16*>(reinterpret_cast<const char*>(p.k) + roff), g);
  load_q(w.vf, reinterpret_cast<const __bf16*>(reinterpret_cast<const char*>(p.v) + roff), g);
  wait_vmcnt<0>();

  DmaLanes<__bf16> dl;
  dma_lanes_init<__bf16>(dl, dil, lane);
  for (int tb = 0; tb < nband; tb += 3) {
    dkv_ring_step<0>(tb, w, c, pol, dl, lse2, dd, st0, st1, st2);
    if (tb + 1 < nband) dkv_ring_step<1>(tb + 1, w, c, pol, dl, lse2, dd, st0, st1, st2);
    if (tb + 2 < nband) dkv_ring_step<2>(tb + 2, w, c, pol, dl, lse2, dd, st0, st1, st2);
  }
  wait_vmcnt<0>();

  if (wave_live) {
    // whole-row stores through the stage of ring step nband, dK then dV (one
    // wave's LDS accesses stay in order)
    const int sa = nband % 3;
    char* slot = (sa == 0 ? st0 : (sa == 1 ? st1 : st2)) + 4096 * wave;
    store_o_rows(slot, reinterpret_cast<char*>(p.dk) + base, w.dk.a, p.scale, lane, kw0, nr, r, dil);
    store_o_rows(slot, reinterpret_cast<char*>(p.dv) + base, w.dv.a, 1.0f, lane, kw0, nr, r, dil);
  }
}

// ----------------------------------------------------------------------------
// Global rows: dQg partials (query blocks over chunks of Kg, Vg, as in the
// forward's global-row blocks). When the block holds fewer than four
// 32-row groups of G, the waves of a group split its 32-key units and their
// partials are summed in LDS.

struct GlobPolSplit {
  GlobPol base;
  int kbeg, sub, wpg;
  DEV bool active(int ku) const { return base.active(ku) && ((ku - kbeg) >> 5) % wpg == sub; }
  DEV bool interior(int ku) const { return base.interior(ku); }
  template <class T> DEV void mask(f32x16& s, int ku, int g) const { base.template mask<T>(s, ku, g); }
};

DEV void bwd_gq_block(const BwdParams& p, int gb, char* st0, char* st1, char* st2) {
  constexpr int ROWB = ElemTraits<__bf16>::ROWB;
  const int tid = threadIdx.x;
  const int lane = tid & 63, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sp = gb % p.nsplit;
  const int grp = (gb / p.nsplit) % p.ngroup;
  const int bh = gb / (p.nsplit * p.ngroup);
  const long base = (long)bh * p.n * ROWB;
  const GSet gs = batch_gset(p.gidx, p.goff, p.ng, bh / p.H);
  if (gs.n <= grp * BAND_WAVES * 32) return;  // no rows of this item's set in this group
  const int qfrags = min(BAND_WAVES, (gs.n + 31) / 32 - grp * BAND_WAVES);
  const int wpg = BAND_WAVES / qfrags;
  const int qbl = wave / wpg, sub = wave % wpg;
  const int qb = grp * BAND_WAVES + qbl;
  const bool live = qbl < qfrags;
  const int gi = qb * 32 + (lane & 31);
  const int pos_q = gs.idx[min(gi, gs.n - 1)];
  const int gmin = gs.idx[min(qb * 32, gs.n - 1)];
  const int gmax = gs.idx[min(grp * BAND_WAVES * 32 + BAND_WAVES * 32 - 1, gs.n - 1)];
  const int k_lo = sp * p.ksplit;
  int k_hi = min(p.n, k_lo + p.ksplit);
  if (p.causal) k_hi = min(k_hi, gmax + 1);
  const int nband = k_hi > k_lo ? (k_hi - k_lo + KT - 1) / KT : 0;

  RingCtx c{(unsigned)(uintptr_t)(lds_void*)st0, (unsigned)(uintptr_t)(lds_void*)st1,
            (unsigned)(uintptr_t)(lds_void*)st2,
            reinterpret_cast<const char*>(p.kg) + base, reinterpret_cast<const char*>(p.vg) + base,
            k_lo, k_hi, nband, 0, 1, wave, lane, g, live, p.c2, {}};
  lds_lanes_init(c.ll, lane);
  const GlobPolSplit pol{{p.causal ? pos_q : 0x7fffffff - 1, k_hi, gmin, p.causal}, k_lo, sub, wpg};
  DqWave w;
  acc2_zero(w.dq);
  if (nband > 0) {
    const long roff = base + (long)pos_q * ROWB;
    ring_start<__bf16>(c);
    load_q(w.qf, reinterpret_cast<const __bf16*>(reinterpret_cast<const char*>(p.qg) + roff), g);
    load_q(w.dof, reinterpret_cast<const __bf16*>(reinterpret_cast<const char*>(p.dout) + roff), g);
    w.lse2 = p.glse2[(long)bh * p.ngp + min(gi, p.ngp - 1)];
    w.dd = p.gdd[(long)bh * p.ngp + min(gi, p.ngp - 1)];
    wait_vmcnt<0>();
    DmaLanes<__bf16> dl;
    dma_lanes_init<__bf16>(dl, 1, lane);
    for (int tb = 0; tb < nband; tb += 3) {
      dq_ring_step<0, true>(tb, w, c, pol, dl, st0, st1, st2);
      if (tb + 1 < nband) dq_ring_step<1, true>(tb + 1, w, c, pol, dl, st0, st1, st2);
      if (tb + 2 < nband) dq_ring_step<2, true>(tb + 2, w, c, pol, dl, st0, st1, st2);
    }
    wait_vmcnt<0>();
  }
  // sum the waves of each row group in LDS, one partial per global row
  __syncthreads();  // the stages are free
  float* W = reinterpret_cast<float*>(wave < 2 ? st0 : st1) + (wave & 1) * 32 * HD;  // [32][64]
#pragma unroll
  for (int dh = 0; dh < 2; ++dh)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      f32x4 t;
#pragma unroll
      for (int e = 0; e < 4; ++e) t[e] = w.dq.a[dh][4 * a + e];
      *reinterpret_cast<f32x4*>(W + (lane & 31) * HD + 32 * dh + 8 * a + 4 * g) = t;
    }
  __syncthreads();
  for (int idx = tid; idx < qfrags * 32 * HD; idx += 256) {
    const int qf = idx / (32 * HD), r = (idx / HD) % 32, d = idx % HD;
    const int row = (grp * BAND_WAVES + qf) * 32 + r;
    if (row >= gs.n) continue;
    float acc = 0.f;
    for (int sw = 0; sw < wpg; ++sw) {
      const int wv = qf * wpg + sw;
      acc += reinterpret_cast<const float*>(wv < 2 ? st0 : st1)[(wv & 1) * 32 * HD + r * HD + d];
    }
    p.part_dqg[(((long)bh * p.ng + row) * p.nsplit + sp) * HD + d] = acc;
  }
}

// ----------------------------------------------------------------------------
// Global rows: dKg, dVg (key blocks over GKV_GROUPS x 128 positions of Kg,
// Vg, one 128-position group after another; the query tiles are the rows of
// G gathered from Qg and dO, loaded once when there are at most 64).

constexpr int GKV_GROUPS = 4;

DEV void bwd_gkv_block(const BwdParams& p, int blk, char* st0, char* st1, int* gpos) {
  constexpr int ROWB = ElemTraits<__bf16>::ROWB;
  constexpr int TILEB = KT * ROWB;
  const int tid = threadIdx.x;
  const int lane = tid & 63, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int span = BM * GKV_GROUPS;
  const int nkb = (p.n + span - 1) / span;
  const int bh = blk / nkb;
  const int kbase = (blk - bh * nkb) * span;
  const GSet gs = batch_gset(p.gidx, p.goff, p.ng, bh / p.H);
  const int ngb = gs.n;
  const long base = (long)bh * p.n * ROWB;
  LdsLanes ll;
  lds_lanes_init(ll, lane);
  const unsigned a0 = (unsigned)(uintptr_t)(lds_void*)st0;
  const char* qb = reinterpret_cast<const char*>(p.qg) + base;
  const char* db = reinterpret_cast<const char*>(p.dout) + base;

  // gather global rows t0 .. t0+63 with their statistics into stage 0
  auto load_tile = [&](int t0, bool first) {
    int gq[4];
    gather_rows(gq, gs.idx, t0, ngb, wave, lane);
    const int gp = gs.idx[min(t0 + lane, ngb - 1)];
    if (!first) __syncthreads();  // the previous tile is consumed
    dma_gather(a0, qb, db, gq, wave, lane);
    const float* src = ((wave & 1) ? p.gdd : p.glse2) + (long)bh * p.ngp + t0 + lane;
    dma4(src, a0 + (unsigned)(2 * TILEB + 256 * wave));
    if (tid < KT) gpos[tid] = gp;
    wait_vmcnt<0>();
    __syncthreads();
  };
  const bool one_tile = ngb <= KT;
  if (one_tile && ngb > 0) load_tile(0, true);

  for (int it = 0; it < GKV_GROUPS; ++it) {
    const int k0 = kbase + it * BM;
    if (k0 >= p.n) break;  // workgroup-uniform
    const int kw0 = k0 + 32 * wave;
    const bool wave_live = kw0 < p.n;
    const int kj = kw0 + (lane & 31);
    const int pos_k = min(kj, p.n - 1);
    const long roff = base + (long)pos_k * ROWB;
    DkvWave w;
    acc2_zero(w.dk);
    acc2_zero(w.dv);
    load_q(w.kf, reinterpret_cast<const __bf16*>(reinterpret_cast<const char*>(p.kg) + roff), g);
    load_q(w.vf, reinterpret_cast<const __bf16*>(reinterpret_cast<const char*>(p.vg) + roff), g);
    for (int t0 = 0; t0 < ngb; t0 += KT) {
      if (!one_tile) load_tile(t0, it == 0 && t0 == 0);
      if (wave_live) {
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          if (t0 + 32 * kh >= ngb) continue;
          dkv_unit(w, st0, kh, ll, p.c2, g, p.causal != 0, [&](f32x16& t) {
            // causal: key position <= the global row's position
#pragma unroll
            for (int j = 0; j < 16; ++j)
              if (pos_k > gpos[32 * kh + key_of_reg<__bf16>(j, g)]) t[j] = -__builtin_inff();
          });
        }
      }
    }
    if (wave_live) {
      // whole-row stores staged in st1, which this block does not use
      char* slot = st1 + 4096 * wave;
      store_o_rows(slot, reinterpret_cast<char*>(p.dkg) + base, w.dk.a, p.scale, lane, kw0, p.n, 0, 1);
      store_o_rows(slot, reinterpret_cast<char*>(p.dvg) + base, w.dv.a, 1.0f, lane, kw0, p.n, 0, 1);
    }
  }
}

// ----------------------------------------------------------------------------
// Global columns: the dK[G], dV[G] terms of the non-global rows whose band
// does not already hold the key (key blocks over query chunks of gcol_qc
// positions; wave w holds global keys 32 (4 kg + w) ..).

struct GcolPol {
  int gpos;      // this lane's global key position
  int gmin;      // smallest global key position of the wave
  int qbeg, qend;  // the query chunk (rows past qend are clamped copies)
  int sub, wpg;  // this wave takes the 32-query units u with u % wpg == sub
  int half, right, dil, causal;
  DEV bool active(int ku) const {
    return ((ku - qbeg) >> 5) % wpg == sub && (!causal || ku + 31 >= gmin);
  }
  DEV bool interior(int) const { return false; }
  template <class T> DEV void mask(f32x16& t, int ku, int g) const {
    if (dil == 1) {  // wave-uniform: no remainder to test
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int qi = ku + key_of_reg<T>(j, g);  // query position
        const int dl = qi - gpos;
        const bool inband = dl >= -right && dl <= half;
        if ((causal && gpos > qi) || inband || qi >= qend) t[j] = -__builtin_inff();
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int qi = ku + key_of_reg<T>(j, g);  // query position
      const int dl = qi - gpos;
      const bool inband = dl >= -right * dil && dl <= half * dil && dl % dil == 0;
      if ((causal && gpos > qi) || inband || qi >= qend) t[j] = -__builtin_inff();
    }
  }
};

DEV void bwd_gcol_block(const BwdParams& p, int blk, char* st0, char* st1, char* st2) {
  constexpr int ROWB = ElemTraits<__bf16>::ROWB;
  const int tid = threadIdx.x;
  const int lane = tid & 63, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ch = blk % p.nchunk;
  const int rest = blk / p.nchunk;
  const int kgb = rest % p.nkgb;
  const int bh = rest / p.nkgb;
  const HeadGeom hg = p.heads[bh % p.H];
  const long base = (long)bh * p.n * ROWB;
  const GSet gs = batch_gset(p.gidx, p.goff, p.ng, bh / p.H);
  if (gs.n <= kgb * BAND_WAVES * 32) return;  // no keys of this item's set in this group
  // The block holds up to four groups of 32 global keys; when it holds fewer,
  // the waves of a group split its query units (wpg waves per group).
  const int kgroups = min(BAND_WAVES, (gs.n + 31) / 32 - kgb * BAND_WAVES);
  const int wpg = BAND_WAVES / kgroups;
  const int kgl = wave / wpg, sub = wave % wpg;
  const int kgi = kgb * BAND_WAVES + kgl;  // this wave's group of 32 global keys
  const bool live = kgl < kgroups;
  const int gi = kgi * 32 + (lane & 31);
  const int gpos = gs.idx[min(gi, gs.n - 1)];
  const int gmin = gs.idx[min(kgi * 32, gs.n - 1)];
  const int qbeg = ch * p.gcol_qc;
  const int qend = min(p.n, qbeg + p.gcol_qc);
  const int nband = (qend - qbeg + KT - 1) / KT;
  const long roff = base + (long)gpos * ROWB;

  RingCtx c{(unsigned)(uintptr_t)(lds_void*)st0, (unsigned)(uintptr_t)(lds_void*)st1,
            (unsigned)(uintptr_t)(lds_void*)st2,
            reinterpret_cast<const char*>(p.q) + base, reinterpret_cast<const char*>(p.dout) + base,
            qbeg, qend, nband, 0, 1, wave, lane, g, live, p.c2, {}};
  lds_lanes_init(c.ll, lane);
  const GcolPol pol{gpos, gmin, qbeg, qend, sub, wpg, hg.half, hg.right, hg.dil, p.causal};
  const float* lse2 = p.lse2 + (long)bh * p.n;
  const float* dd = p.dd + (long)bh * p.n;

  DkvWave w;
  acc2_zero(w.dk);
  acc2_zero(w.dv);
  dma_tile<__bf16>(c.a0, c.kb, c.vb, qbeg, qend, 0, 1, wave, lane);
  dma_stats(c.a0, lse2, dd, qbeg, qend, 0, 1, wave, lane);
  const int q1 = qbeg + min(1, nband - 1) * KT;
  dma_tile<__bf16>(c.a1, c.kb, c.vb, q1, qend, 0, 1, wave, lane);
  dma_stats(c.a1, lse2, dd, q1, qend, 0, 1, wave, lane);
  load_q(w.kf, reinterpret_cast<const __bf16*>(reinterpret_cast<const char*>(p.k) + roff), g);
  load_q(w.vf, reinterpret_cast<const __bf16*>(reinterpret_cast<const char*>(p.v) + roff), g);
  wait_vmcnt<0>();
  DmaLanes<__bf16> dl;
  dma_lanes_init<__bf16>(dl, 1, lane);
  for (int tb = 0; tb < nband; tb += 3) {
    dkv_ring_step<0>(tb, w, c, pol, dl, lse2, dd, st0, st1, st2);
    if (tb + 1 < nband) dkv_ring_step<1>(tb + 1, w, c, pol, dl, lse2, dd, st0, st1, st2);
    if (tb + 2 < nband) dkv_ring_step<2>(tb + 2, w, c, pol, dl, lse2, dd, st0, st1, st2);
  }
  wait_vmcnt<0>();
  // Sum the partials of the waves of each key group in LDS (dK, then dV) and
  // write one per global key.
  __syncthreads();  // the stages are free
  for (int which = 0; which < 2; ++which) {
    const Acc2& a = which ? w.dv : w.dk;
    float* W = reinterpret_cast<float*>(wave < 2 ? st0 : st1) + (wave & 1) * 32 * HD;  // [32][64]
    const int row = lane & 31;
#pragma unroll
    for (int dh = 0; dh < 2; ++dh)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4 t;
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = a.a[dh][4 * q + e];
        *reinterpret_cast<f32x4*>(W + row * HD + 32 * dh + 8 * q + 4 * g) = t;
      }
    __syncthreads();
    for (int idx = tid; idx < kgroups * 32 * HD; idx += 256) {
      const int kg = idx / (32 * HD), r = (idx / HD) % 32, d = idx % HD;
      const int gk = (kgb * BAND_WAVES + kg) * 32 + r;
      if (gk >= gs.n) continue;
      float acc = 0.f;
      for (int sw = 0; sw < wpg; ++sw) {
        const int wv = kg * wpg + sw;
        acc += reinterpret_cast<const float*>(wv < 2 ? st0 : st1)[(wv & 1) * 32 * HD + r * HD + d];
      }
      p.part_gkv[(((long)bh * p.nchunk + ch) * p.ng32 + gk) * (2 * HD) + which * HD + d] = acc;
    }
    __syncthreads();
  }
}

// ----------------------------------------------------------------------------
// One global token per item, streamed. The global row and the global column
// are a single row against all n positions: the matrix cores would compute
// 32 rows for the one that exists, so these blocks stream the n positions
// through registers instead, four lanes per position (lane % 4 holds the
// features 16 (lane % 4) .. +15), with fp32 dot products of bf16 pairs and
// fp32 sums; with 16 features per lane the registers hold many positions,
// and each wave keeps SDEPTH rounds of 16 positions in flight. Round it of
// wave w: positions p0 + 16 (4 it + w) + (lane / 4).

typedef unsigned u32x4s __attribute__((ext_vector_type(4)));
constexpr int SLPK = 4;            // lanes per position
constexpr int SDPL = HD / SLPK;    // features per lane
constexpr int SCH = SDPL * 2 / 16; // 16-byte pieces of a lane's features
constexpr int SKPW = 64 / SLPK;    // positions per wave and round
// rounds in flight per wave (bwd_main runs two waves per SIMD, so the
// registers are there)
constexpr int SDEPTH = 8;

// this lane's 16 features of one row, as 8 bf16 pairs
DEV void load_part(u32x4s (&x)[SCH], const char* row, int part) {
#pragma unroll
  for (int c = 0; c < SCH; ++c) x[c] = *reinterpret_cast<const u32x4s*>(row + part * (2 * SDPL) + 16 * c);
}
// the full 64-feature dot product of two rows held in parts by 4 lanes
DEV float dot_parts(const u32x4s (&a)[SCH], const u32x4s (&b)[SCH]) {
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < SCH; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // the elements go through values: a bit cast of a vector element
      // expression itself reads the vector's first element
      const unsigned ua = a[c][e], ub = b[c][e];
      s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, ua), __builtin_bit_cast(bf16x2, ub), s, false);
    }
  s += __shfl_xor(s, 1);
  return s + __shfl_xor(s, 2);
}
DEV float bf_lo(unsigned u) { return __builtin_bit_cast(float, u << 16); }
DEV float bf_hi(unsigned u) { return __builtin_bit_cast(float, u & 0xffff0000u); }
// acc[i] += f * x[i] over this lane's features
DEV void axpy_part(float (&acc)[SDPL], float f, const u32x4s (&x)[SCH]) {
#pragma unroll
  for (int c = 0; c < SCH; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[8 * c + 2 * e] = __builtin_fmaf(f, bf_lo(x[c][e]), acc[8 * c + 2 * e]);
      acc[8 * c + 2 * e + 1] = __builtin_fmaf(f, bf_hi(x[c][e]), acc[8 * c + 2 * e + 1]);
    }
}
// f * x over this lane's features, rounded to bf16
DEV void scale_part(u32x4s (&t)[SCH], float f, const u32x4s (&x)[SCH]) {
#pragma unroll
  for (int c = 0; c < SCH; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bf16x2 h{(__bf16)(f * bf_lo(x[c][e])), (__bf16)(f * bf_hi(x[c][e]))};
      t[c][e] = __builtin_bit_cast(unsigned, h);
    }
}
// The wave's 16 rows (the 4 lanes of position kq holding row key0 + kq in
// 32-byte parts) staged in the wave's 2 KB of LDS and written out as whole
// 128-byte rows, eight lanes per row, with non-temporal stores (rows >= kend
// skipped). The same wave reads what it wrote, so no barrier is needed.
DEV void store_rows_nt(char* w2k, const u32x4s (&t)[SCH], int kq, int part, char* dst, int key0, int kend) {
  typedef __attribute__((address_space(3))) char lds_char;
  typedef __attribute__((address_space(3))) u32x4s lds_u32x4;
  lds_char* sb = (lds_char*)w2k;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int c = 0; c < SCH; ++c) *(lds_u32x4*)(sb + kq * 128 + 16 * ((SCH * part + c) ^ (kq & 7))) = t[c];
#pragma unroll
  for (int k = 0; k < SKPW / 8; ++k) {
    const int row = 8 * k + (lane >> 3), ch = lane & 7;
    const u32x4s v = *(lds_u32x4*)(sb + row * 128 + 16 * (ch ^ (row & 7)));
    if (key0 + row < kend)
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4s*>(dst + (long)(key0 + row) * 128 + 16 * ch));
  }
}
// Sum acc (this lane's features of position kq) over the block's 4 x SKPW
// positions into *out (feature t of the first wave, t < 64), through st0 as
// [wave][SKPW][64] floats with 16-byte chunks swizzled by the position, then
// [4][64] wave sums.
DEV void fold_parts(const float (&acc)[SDPL], char* st0, float* out) {
  typedef __attribute__((address_space(3))) char lds_char;
  typedef __attribute__((address_space(3))) float lds_float;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int part = lane % SLPK, kq = lane / SLPK;
  lds_char* wb = (lds_char*)(st0 + wave * (SKPW * 256));
  __syncthreads();  // the buffers are free
#pragma unroll
  for (int c = 0; c < SDPL / 4; ++c) {
    f32x4 t;
#pragma unroll
    for (int e = 0; e < 4; ++e) t[e] = acc[4 * c + e];
    *reinterpret_cast<__attribute__((address_space(3))) f32x4*>(wb + kq * 256 + part * (4 * SDPL) +
                                                                 16 * (c ^ (kq % (SDPL / 4)))) = t;
  }
  __syncthreads();
  // thread t: feature t % 64 over the positions of wave t / 64
  const int d = lane, pd = d / SDPL, c = (d % SDPL) / 4;
  float sum = 0.f;
#pragma unroll
  for (int k = 0; k < SKPW; ++k)
    sum += *(const lds_float*)(wb + k * 256 + pd * (4 * SDPL) + 16 * (c ^ (k % (SDPL / 4))) + 4 * (d % 4));
  __syncthreads();
  lds_float* red = (lds_float*)(lds_char*)st0;  // [4][64]
  red[wave * HD + d] = sum;
  __syncthreads();
  if (tid < HD) *out = red[tid] + red[HD + tid] + red[2 * HD + tid] + red[3 * HD + tid];
  __syncthreads();
}

// The global row of (b, h) against one chunk of keys: dKg and dVg of every
// key of the chunk (zero where the row does not attend: past it when causal,
// or everywhere in an item without a global token) and the chunk's dQg
// partial (unscaled), which bwd_gred sums.
DEV void bwd_grow_stream(const BwdParams& p, int blk, char* st0) {
  constexpr int ROWB = ElemTraits<__bf16>::ROWB;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int part = lane % SLPK, kq = lane / SLPK;
  const int sp = blk % p.nsplit, bh = blk / p.nsplit;
  const int k_lo = sp * p.ksplit, k_end = min(p.n, k_lo + p.ksplit);
  const long base = (long)bh * p.n * ROWB;
  const char* kgb = reinterpret_cast<const char*>(p.kg) + base;
  const char* vgb = reinterpret_cast<const char*>(p.vg) + base;
  char* dkgb = reinterpret_cast<char*>(p.dkg) + base;
  char* dvgb = reinterpret_cast<char*>(p.dvg) + base;
  const int nit = (k_end - k_lo + 4 * SKPW - 1) / (4 * SKPW);
  auto key = [&](int it) { return k_lo + SKPW * (4 * it + wave) + kq; };
  auto fetch = [&](int it, u32x4s (&kk)[SCH], u32x4s (&vv)[SCH]) {
    const long j = min(key(it), k_end - 1);
    load_part(kk, kgb + j * ROWB, part);
    load_part(vv, vgb + j * ROWB, part);
  };
  u32x4s kbuf[SDEPTH][SCH], vbuf[SDEPTH][SCH];
#pragma unroll
  for (int s = 0; s < SDEPTH; ++s)
    if (s < nit) fetch(s, kbuf[s], vbuf[s]);
  const GSet gs = batch_gset(p.gidx, p.goff, p.ng, bh / p.H);
  const bool has = gs.n > 0;  // workgroup-uniform
  const int pos = has ? gs.idx[0] : 0;
  const int k_att = !has ? k_lo : (p.causal ? min(k_end, pos + 1) : k_end);  // keys < k_att attend
  u32x4s qg[SCH], dog[SCH];
  float lse2 = __builtin_inff(), dd = 0.f;
  if (has) {
    load_part(qg, reinterpret_cast<const char*>(p.qg) + base + (long)pos * ROWB, part);
    load_part(dog, reinterpret_cast<const char*>(p.dout) + base + (long)pos * ROWB, part);
    lse2 = p.glse2[(long)bh * p.ngp];
    dd = p.gdd[(long)bh * p.ngp];
  } else {
#pragma unroll
    for (int c = 0; c < SCH; ++c) { qg[c] = u32x4s{0u, 0u, 0u, 0u}; dog[c] = qg[c]; }
  }
  float dq[SDPL];
#pragma unroll
  for (int i = 0; i < SDPL; ++i) dq[i] = 0.f;
  char* w2k = st0 + 2048 * wave;
  auto step = [&](int it, const u32x4s (&kk)[SCH], const u32x4s (&vv)[SCH]) {
    const int j = key(it);
    const float s = dot_parts(qg, kk);
    const float dp = dot_parts(dog, vv);
    const float pr = j < k_att ? __builtin_amdgcn_exp2f(s * p.c2 - lse2) : 0.f;
    const float ds = pr * (dp - dd);
    axpy_part(dq, ds, kk);
    u32x4s t[SCH];
    scale_part(t, ds * p.scale, qg);
    store_rows_nt(w2k, t, kq, part, dkgb, j - kq, k_end);
    scale_part(t, pr, dog);
    store_rows_nt(w2k, t, kq, part, dvgb, j - kq, k_end);
  };
  for (int it0 = 0; it0 < nit; it0 += SDEPTH) {
#pragma unroll
    for (int s = 0; s < SDEPTH; ++s) {
      const int it = it0 + s;
      if (it < nit) {
        step(it, kbuf[s], vbuf[s]);
        if (it + SDEPTH < nit) fetch(it + SDEPTH, kbuf[s], vbuf[s]);
      }
    }
  }
  if (!has) return;  // workgroup-uniform: no dQg partial for an item without G
  float out = 0.f;
  fold_parts(dq, st0, &out);
  if (tid < HD) p.part_dqg[(((long)bh * p.ng + 0) * p.nsplit + sp) * HD + tid] = out;
}

// The global column of (b, h) against one chunk of query rows: the dK[g],
// dV[g] terms (unscaled dK) of the rows that attend to the global key g
// from outside their band (rows of G have LSE +inf, so P = 0), one partial
// per chunk for bwd_gred.
DEV void bwd_gcol_stream(const BwdParams& p, int blk, char* st0) {
  constexpr int ROWB = ElemTraits<__bf16>::ROWB;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int part = lane % SLPK, kq = lane / SLPK;
  const int ch = blk % p.nchunk, bh = blk / p.nchunk;
  const int qbeg = ch * p.gcol_qc, qend = min(p.n, qbeg + p.gcol_qc);
  const long base = (long)bh * p.n * ROWB;
  const char* qb = reinterpret_cast<const char*>(p.q) + base;
  const char* db = reinterpret_cast<const char*>(p.dout) + base;
  const float* lse2 = p.lse2 + (long)bh * p.n;
  const float* ddr = p.dd + (long)bh * p.n;
  const int nit = (qend - qbeg + 4 * SKPW - 1) / (4 * SKPW);
  auto row = [&](int it) { return qbeg + SKPW * (4 * it + wave) + kq; };
  auto fetch = [&](int it, u32x4s (&qq)[SCH], u32x4s (&oo)[SCH], float& l2, float& d) {
    const long i = min(row(it), qend - 1);
    load_part(qq, qb + i * ROWB, part);
    load_part(oo, db + i * ROWB, part);
    l2 = lse2[i];
    d = ddr[i];
  };
  u32x4s qbuf[SDEPTH][SCH], obuf[SDEPTH][SCH];
  float lbuf[SDEPTH], dbuf[SDEPTH];
#pragma unroll
  for (int s = 0; s < SDEPTH; ++s)
    if (s < nit) fetch(s, qbuf[s], obuf[s], lbuf[s], dbuf[s]);
  const GSet gs = batch_gset(p.gidx, p.goff, p.ng, bh / p.H);
  if (gs.n == 0) return;  // workgroup-uniform: no global key in this item
  const int gpos = gs.idx[0];
  const HeadGeom hg = p.heads[bh % p.H];
  u32x4s kg[SCH], vg[SCH];
  load_part(kg, reinterpret_cast<const char*>(p.k) + base + (long)gpos * ROWB, part);
  load_part(vg, reinterpret_cast<const char*>(p.v) + base + (long)gpos * ROWB, part);
  float dk[SDPL], dv[SDPL];
#pragma unroll
  for (int i = 0; i < SDPL; ++i) { dk[i] = 0.f; dv[i] = 0.f; }
  auto step = [&](int it, const u32x4s (&qq)[SCH], const u32x4s (&oo)[SCH], float l2, float d) {
    const int i = row(it);
    const int dl = i - gpos;  // the row holds g in its band iff g is a band key of it
    const bool inband = dl >= -hg.right * hg.dil && dl <= hg.half * hg.dil && dl % hg.dil == 0;
    const bool ok = i < qend && !inband && !(p.causal && gpos > i);
    const float s = dot_parts(qq, kg);
    const float dp = dot_parts(oo, vg);
    const float pr = ok ? __builtin_amdgcn_exp2f(s * p.c2 - l2) : 0.f;  // l2 = +inf on rows of G
    const float ds = pr * (dp - d);
    axpy_part(dk, ds, qq);
    axpy_part(dv, pr, oo);
  };
  for (int it0 = 0; it0 < nit; it0 += SDEPTH) {
#pragma unroll
    for (int s = 0; s < SDEPTH; ++s) {
      const int it = it0 + s;
      if (it < nit) {
        step(it, qbuf[s], obuf[s], lbuf[s], dbuf[s]);
        if (it + SDEPTH < nit) fetch(it + SDEPTH, qbuf[s], obuf[s], lbuf[s], dbuf[s]);
      }
    }
  }
  float outk = 0.f, outv = 0.f;
  fold_parts(dk, st0, &outk);
  fold_parts(dv, st0, &outv);
  if (tid < HD) {
    float* rec = p.part_gkv + (((long)bh * p.nchunk + ch) * p.ng32 + 0) * (2 * HD);
    rec[tid] = outk;
    rec[HD + tid] = outv;
  }
}

// ----------------------------------------------------------------------------
// Reduction for the global tokens, after bwd_main: one block per (b*h, global
// row). dqg[g] = s * sum of the chunk partials; dk[g], dv[g] gain the
// global-column terms of every query chunk.

__global__ __launch_bounds__(256) void bwd_gred(BwdParams p) {
  const int gi = blockIdx.x % p.ng;
  const long bh = blockIdx.x / p.ng;
  const GSet gs = batch_gset(p.gidx, p.goff, p.ng, (int)(bh / p.H));
  if (gi >= gs.n) return;
  const int t = threadIdx.x, d = t & 63, part = t >> 6;
  const long row = bh * p.n + gs.idx[gi];
  // sum `count` partials `stride` floats apart, eight loads in flight at once
  auto sum = [](const float* src, int count, long stride) {
    float acc = 0.f;
    for (int c0 = 0; c0 < count; c0 += 8) {
      float x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = c0 + i < count ? src[(c0 + i) * stride] : 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc += x[i];
    }
    return acc;
  };
  if (part == 0) {
    const float acc = sum(p.part_dqg + ((bh * p.ng + gi) * p.nsplit) * HD + d, p.nsplit, HD);
    reinterpret_cast<__bf16*>(p.dqg)[row * HD + d] = (__bf16)(acc * p.scale);
  } else if (part <= 2) {
    const int off = part == 1 ? 0 : HD;
    __bf16* dst = reinterpret_cast<__bf16*>(part == 1 ? p.dk : p.dv) + row * HD + d;
    const float band = (float)*dst;
    const float acc = sum(p.part_gkv + ((bh * p.nchunk) * p.ng32 + gi) * (2 * HD) + off + d,
                          p.nchunk, (long)p.ng32 * 2 * HD);
    *dst = (__bf16)(band + (part == 1 ? acc * p.scale : acc));
  }
}

// ----------------------------------------------------------------------------
// The main backward kernel: the global-token blocks first (global-column
// partials, dQg partials, dKg/dVg), then the band query blocks (dq) and the
// band key blocks (dk, dv) over the same tile schedule, the two blocks of a
// tile next to each other. The band blocks take
// several rounds of workgroup slots, so the long, mostly serial global-token
// blocks start at once and the band blocks pack around them (on the encoder
// workload 117.5 us instead of 133 us with them last).

// Two instantiations: GSTREAM = true for plans with one global token per
// item (the streamed global row and column), false for every other plan, so
// that the streaming code does not enlarge the kernel that the others run.
template <bool GSTREAM>
__global__ __launch_bounds__(256, 2) void bwd_main(BwdParams p) {
  __shared__ __attribute__((aligned(1024))) char st0[QSTAGEB];
  __shared__ __attribute__((aligned(1024))) char st1[QSTAGEB];
  __shared__ __attribute__((aligned(1024))) char st2[QSTAGEB];
  __shared__ int gmeta[2][KT];
  int b = blockIdx.x;
  if (b < p.n_gcol) {
    if constexpr (GSTREAM) bwd_gcol_stream(p, b, st0);
    else bwd_gcol_block(p, b, st0, st1, st2);
    return;
  }
  b -= p.n_gcol;
  if (b < p.n_gq) {
    if constexpr (GSTREAM) bwd_grow_stream(p, b, st0);
    else bwd_gq_block(p, b, st0, st1, st2);
    return;
  }
  b -= p.n_gq;
  if constexpr (!GSTREAM) {
    if (b < p.n_gkv) { bwd_gkv_block(p, b, st0, st1, gmeta[0]); return; }
    b -= p.n_gkv;
  }
  // The query and key blocks of a tile are neighbours in the order: a tile's
  // K and V rows (the query blocks' ring tiles, the key block's own rows)
  // and its Q and dO rows (the other way round) then meet in one XCD's L2 at
  // about the same time, instead of being fetched once by the query blocks
  // and again by the key blocks a round later.
  const int lb = xcd_remap(b, 2 * p.nq);
  if ((lb & 1) == 0) bwd_dq_block(p, lb >> 1, st0, st1, st2, gmeta);
  else bwd_dkv_block(p, lb >> 1, st0, st1, st2);
}

}  // namespace swattn
