// Device kernels of the banded sliding-window attention forward pass (gfx950).
//
// Operation (Longformer summary page, section 3-1 "Attention Pattern", and
// section 7 for the left-only mask): row i of head h attends to the keys
// i + k*dil_h, k in [-w_h/2, R_h] (R_h = 0 when causal, else w_h/2), plus
// every global token (left of i when causal), each key once; rows of the
// global tokens attend to every key through the separate projections Qg, Kg,
// Vg. Softmax scale 1/sqrt(64).
//
// Work decomposition (all kernels share the wave-level 32-key unit below):
//  * band blocks: one workgroup = 4 waves = 128 query rows of one residue class
//    r (rows r, r+dil, r+2*dil, ... of one (batch, head)); within a residue
//    class the dilated window is an ordinary window of w+1 keys, so K/V rows
//    are read with a row stride of dil*64 elements and no key is wasted on
//    the gaps. Key tiles of 64 rows stream through a 3-stage LDS ring filled
//    by direct global->LDS loads, shared by the 4 waves; each wave skips the
//    32-key units that lie outside its own 32 rows' band. The global columns
//    are extra key tiles gathered from K[G], V[G], masked so that a global key
//    already inside the band is not counted twice; the running max/sum of
//    the online softmax merges them with the band exactly as a log-sum-exp
//    merge would.
//  * global-row blocks: rows of G against a chunk of all keys with Qg, Kg,
//    Vg, through the same ring; each writes an unnormalised partial (o, m, l)
//    per chunk. They share one launch (attn_fwd) with the band blocks and
//    come after them in the grid.
//  * global_rows_merge: log-sum-exp merge of the chunks; overwrites rows G of
//    O (and LSE), stream-ordered after attn_fwd.
//
// Score tiles are computed transposed, S^T = K Q^T, with the 32x32 MFMA: each
// lane then owns one query column, so row max and row sum are in-lane
// reductions plus one exchange with the lane 32 apart. K rows are fed to the
// MFMA in a permuted order (bits 2 and 3 of the row index swapped) so that
// the accumulator registers come out in exactly the B-operand layout of the
// following P V MFMA: P never leaves registers. V stays row-major in LDS and
// is read transposed with ds_read_b64_tr_b16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

#define DEV __device__ __forceinline__

constexpr int HD = 64;        // head dimension
constexpr int KT = 64;        // keys per LDS tile
constexpr int BAND_WAVES = 4; // waves per band workgroup
constexpr int BM = 32 * BAND_WAVES;  // query rows per band workgroup
constexpr int NEG_SENTINEL = -(1 << 30);
constexpr float LOG2E = 1.4426950408889634f;

// One band workgroup: (batch*head, residue class r, first residue-local
// query row q0, rows nr of the residue class) and the head's band geometry,
// read with one 32-byte scalar load.
struct TileRec {
  int bh, r, q0, nr;
  int half;   // w/2, clipped to n
  int right;  // 0 when causal, else half
  int dil;    // dilation, clipped to n
  int pad;
};

struct BandParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  // band workgroups: an explicit list, or NULL when every head has the same
  // geometry (uni_*): then block b is (bh, r, q-block) = b in mixed radix
  // (B*H, uni_dil, uni_nqb)
  const TileRec* tiles;
  int uni_half, uni_right, uni_dil, uni_nqb;
  const int* gidx;       // sorted G: one set, or the batch items' sets one after another
  const int* goff;       // [B+1] offsets of the per-item sets in gidx, or NULL (one set)
  int ng;                // |G| (one set), or the largest per-item |G|
  // key split: each band tile's key tiles are shared out over `parts`
  // workgroups that write unnormalised partials (o[64], m, l) to
  // part[(b*h*n + position) * parts + k][68] for band_merge (parts = 1: none)
  int parts;
  float* part;
  int fair;     // progress-based wave priorities (no global-row blocks in the launch)
  int gskip;    // 1: leave the rows of G alone (the global-row blocks write them)
  int H;
  int n;
  int causal;
  float c2;     // scale * log2(e)
  float scale;  // 1/sqrt(64)
};

constexpr int PART_STRIDE = 68;  // floats per partial record: o[64], m, l, 2 pad
constexpr int MAX_KEY_SPLIT = 16;

struct GlobalParams {
  const void* qg;
  const void* kg;
  const void* vg;
  void* o;
  float* lse;
  const int* gidx;
  const int* goff;  // as in BandParams
  int H;
  float* part_o;  // [BH][ng][nsplit][64]
  float* part_ml; // [BH][ng][nsplit][2]  (max, sum)
  int ng;
  int n;
  int causal;
  int nsplit;
  int ksplit;   // keys per split, multiple of 64
  int nqb;      // ceil(ng / 32): blocks of 32 global rows
  int ngroup;   // ceil(nqb / 4): groups of 4 such blocks (one per wave)
  int stream;   // 1: global_row_stream blocks (bf16, at most one global token per item)
  int fuse;     // with stream: the chunks' last block folds them (no global_rows_merge)
  int* gcount;  // [B*H] arrival counters for fuse, zero between launches
  float c2;
  float scale;
};

// The global tokens of batch item b: the shared set, or the b-th per-item
// set (its size may be anything up to ng, 0 included).
struct GSet {
  const int* idx;
  int n;
};
DEV GSet batch_gset(const int* gidx, const int* goff, int ng, int b) {
  if (!goff) return GSet{gidx, ng};
  const int o0 = goff[b];
  return GSet{gidx + o0, goff[b + 1] - o0};
}

// ----------------------------------------------------------------------------
// small helpers

// XCD-aware block order: consecutive hardware block ids go round-robin to the
// 8 XCDs; give each XCD a contiguous range of logical tiles so that tiles
// sharing K/V rows share one L2.
DEV int xcd_remap(int bid, int nblocks) {
  constexpr int NX = 8;
  int per = (nblocks + NX - 1) / NX;
  int tall = nblocks % NX == 0 ? NX : nblocks % NX;
  int x = bid % NX, loc = bid / NX;
  return x < tall ? x * per + loc : tall * per + (x - tall) * (per - 1) + loc;
}

// 16-byte-chunk swizzle of a 128-byte LDS row: keeps the K-operand reads
// (16 lanes, rows pi(0..15), one chunk) and the transposed V reads (4 rows x
// 2 chunks per 16 lanes) free of bank conflicts.
DEV int swz(int row) {
  return (((row >> 1) & 1) << 2) | ((row >> 2) & 1) | (((row >> 3) & 1) << 1);
}

// MFMA row r of the S^T tile -> key within the 32-key unit (swap bits 2, 3).
DEV int kperm16(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }
// fp32 variant: MFMA row r = 8a + 4g + b -> key 8a + 2b + g.
DEV int kperm32(int r) { return (r & ~7) | ((r & 3) << 1) | ((r >> 2) & 1); }

// key (within the 32-key unit) held by accumulator register j of lane group g
DEV constexpr int key_of_reg16(int j, int g) { return ((j >> 3) << 4) + (g << 3) + (j & 7); }
DEV constexpr int key_of_reg32(int j, int g) { return 2 * j + g; }

DEV f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
DEV f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Values of lane l and lane l^32, returned as (lo-half copy, hi-half copy):
// max/sum of the two is the pair's max/sum on every lane.
DEV f32x2 pair_swap(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return f32x2{__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1])};
}
DEV float pair_max(float x) { const f32x2 t = pair_swap(x); return fmaxf(t[0], t[1]); }
DEV float pair_sum(float x) { const f32x2 t = pair_swap(x); return t[0] + t[1]; }

// A workgroup barrier that does not wait for outstanding global->LDS loads
// (the loads of the next tiles stay in flight); the asm statements keep the
// compiler from moving memory accesses across it.
DEV void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// Wait until at most N vector-memory loads of this wave are outstanding.
template <int N> DEV void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 0xf) | (0x7 << 4) | (0xf << 8) | ((N >> 4) << 14));
  asm volatile("" ::: "memory");
}

template <class T> struct ElemTraits;
template <> struct ElemTraits<__bf16> {
  static constexpr int ROWB = 128;           // bytes per K/V row
  static constexpr int CPR = ROWB / 16;      // 16-byte chunks per row
  static DEV int phys(int row, int ch) { return ch ^ swz(row); }  // involution
  static DEV int lds_off(int row, int ch) { return row * ROWB + (phys(row, ch) << 4); }
};
template <> struct ElemTraits<float> {
  static constexpr int ROWB = 256;
  static constexpr int CPR = ROWB / 16;
  static DEV int phys(int, int ch) { return ch; }
  static DEV int lds_off(int row, int ch) { return row * ROWB + (ch << 4); }
};

// ----------------------------------------------------------------------------
// Wave-level engine.
//
// State of one wave: 32 query rows (lane l and lane l^32 share row l%32),
// reference max m (raw score units; the same on both lanes of a row), this
// lane's partial row sum l, and O^T accumulators for the two 32-wide halves
// of d.
template <class T> struct QFrag;
template <> struct QFrag<__bf16> { bf16x8 v[4]; };  // d = 16s + 8g + e
template <> struct QFrag<float> { float v[32]; };   // d = 2s + g

struct WaveAcc {
  f32x16 o[2];
  float m;     // reference max (raw score units)
  float l;     // this lane's partial row sum
  float thr;   // m + RESCALE_LOG2 / c2: a unit max above it raises m
  float moff;  // -m * c2 (0 while m = -inf): exp2 argument offset
};

DEV void acc_init(WaveAcc& a) {
#pragma unroll
  for (int i = 0; i < 16; ++i) { a.o[0][i] = 0.f; a.o[1][i] = 0.f; }
  a.m = -__builtin_inff();
  a.l = 0.f;
  a.thr = -__builtin_inff();
  a.moff = 0.f;
}

// Load the B operand of S^T = K Q^T for this lane's query row (global memory).
DEV void load_q(QFrag<__bf16>& qf, const __bf16* row, int g) {
  const uint4* p = reinterpret_cast<const uint4*>(row);
#pragma unroll
  for (int s = 0; s < 4; ++s) qf.v[s] = __builtin_bit_cast(bf16x8, p[2 * s + g]);
}
DEV void load_q(QFrag<float>& qf, const float* row, int g) {
#pragma unroll
  for (int s = 0; s < 32; ++s) qf.v[s] = row[2 * s + g];
}

// fp32 path: S^T for one 32-key unit (rows 32*kh .. 32*kh+31 of the LDS tile).
DEV f32x16 score_unit(const char* kbuf, int kh, const QFrag<float>& qf, int lane) {
  const int g = lane >> 5;
  const int row = kperm32(lane & 31) + 32 * kh;
  const float* kr = reinterpret_cast<const float*>(kbuf + row * ElemTraits<float>::ROWB);
  f32x16 s = {};
#pragma unroll
  for (int st = 0; st < 32; ++st) s = mfma_f32(kr[2 * st + g], qf.v[st], s);
  return s;
}

// fp32 path: O^T += V^T P^T for one 32-key unit.
DEV void pv_unit(WaveAcc& acc, const char* vbuf, int kh, const f32x16& p, int lane) {
  const int g = lane >> 5;
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    const float* vr = reinterpret_cast<const float*>(vbuf + (32 * kh + 2 * t + g) * ElemTraits<float>::ROWB);
#pragma unroll
    for (int dh = 0; dh < 2; ++dh) acc.o[dh] = mfma_f32(vr[32 * dh + (lane & 31)], p[t], acc.o[dh]);
  }
}

// key_of_reg(j, g) = key_reg_base(j) + g * key_g_step: masks compare against
// bounds shifted by the lane's group, so the per-register offsets stay
// immediates instead of occupying VGPRs.
template <class T> DEV constexpr int key_reg_base(int j) {
  if constexpr (sizeof(T) == 2) return ((j >> 3) << 4) + (j & 7);
  else return 2 * j;
}
template <class T> constexpr int key_g_step = sizeof(T) == 2 ? 8 : 1;

template <class T> DEV constexpr int key_of_reg(int j, int g) {
  if constexpr (sizeof(T) == 2) return key_of_reg16(j, g);
  else return key_of_reg32(j, g);
}

// Online-softmax update and P V for one 32-key unit whose raw scores are s
// (masked entries at -inf).
//
// The reference max m is raised only when a row's unit max exceeds it by more
// than RESCALE_LOG2 in the exp2 domain (then O and l are rescaled, and both
// lanes of the row agree on the new m); otherwise probabilities relative to
// the stale m stay below 2^RESCALE_LOG2, which fp32 accumulators and the bf16
// P operand hold without loss of relative precision. O = acc / l and
// LSE = m*scale + ln l are the same quantities as with an exact running max.
// In bf16 the P V product takes the weights rounded to bf16 while the row
// sum l adds the unrounded fp32 weights, so LSE carries fp32 rounding only
// and O the bf16 rounding of each weight (relative 2^-9), which averages
// out over the row.
constexpr float RESCALE_LOG2 = 8.0f;

// fp32 path: online softmax of one 32-key unit and O += P V.
DEV void softmax_pv_unit(WaveAcc& acc, f32x16 s, const char* vbuf, int kh, int lane, float c2) {
  float mx = s[0];
#pragma unroll
  for (int j = 1; j < 16; ++j) mx = fmaxf(mx, s[j]);
  if (__builtin_amdgcn_ballot_w64(mx > acc.thr)) {
    const float pm = pair_max(mx);
    const bool upd = pm > acc.thr;  // the same decision on both lanes of a row
    // rows that do not move keep alpha = 1 (also while their m is still -inf)
    const float alpha = upd ? __builtin_amdgcn_exp2f((acc.m - pm) * c2) : 1.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) { acc.o[0][i] *= alpha; acc.o[1][i] *= alpha; }
    acc.l *= alpha;
    acc.m = upd ? pm : acc.m;
    acc.thr = acc.m + RESCALE_LOG2 / c2;
    // a row with every key masked so far has m = -inf and only -inf scores
    acc.moff = acc.m == -__builtin_inff() ? 0.f : -acc.m * c2;
  }
  float l0 = 0.f, l1 = 0.f;
#pragma unroll
  for (int j = 0; j < 16; j += 2) {
    s[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j], c2, acc.moff));
    s[j + 1] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j + 1], c2, acc.moff));
    l0 += s[j];
    l1 += s[j + 1];
  }
  acc.l += l0 + l1;
  pv_unit(acc, vbuf, kh, s, lane);
}

// bf16 path: the pieces of a 32-key unit as the ring uses them. The K and V
// fragments are read from LDS into registers ahead of the MFMAs (the V reads
// are in flight during the softmax).
struct KFrag { bf16x8 v[4]; };      // A operand of S^T, 4 k-steps of 16 d
struct VFrag { bf16x8 a[2][2]; };   // A operand of O^T, [16-key step][d half]
struct PFrag { bf16x8 b[2]; };      // B operand of O^T, [16-key step]

// Lane-dependent byte offsets of the bf16 fragment reads within a tile. The
// swizzle only permutes 16-byte chunks inside a 128-byte row and depends on
// row bits 1..3, so the unit (32 rows) and the 16-key step (16 rows) enter as
// plain byte offsets; what differs per lane is kept here, once per wave:
//   k[st]     K operand, k-step st (chunk 2*st + g of row kperm16(lane%32))
//   v[w][dh]  transposed V read w (rows +0 / +4) of d half dh
struct LdsLanes { int k[4]; int v[2][2]; };

DEV void lds_lanes_init(LdsLanes& ll, int lane) {
  const int g = lane >> 5;
  const int row = kperm16(lane & 31);
#pragma unroll
  for (int st = 0; st < 4; ++st) ll.k[st] = ElemTraits<__bf16>::lds_off(row, 2 * st + g);
  const int i16 = lane & 15;
#pragma unroll
  for (int w = 0; w < 2; ++w)
#pragma unroll
    for (int dh = 0; dh < 2; ++dh) {
      const int col = 32 * dh + 16 * ((lane >> 4) & 1) + 4 * (i16 & 3);
      const int row0 = 8 * g + (i16 >> 2) + 4 * w;
      ll.v[w][dh] = ElemTraits<__bf16>::lds_off(row0, col >> 3) + ((col & 7) << 1);
    }
}

DEV KFrag load_kfrag(const char* kbuf, int kh, const LdsLanes& ll) {
  KFrag k;
#pragma unroll
  for (int st = 0; st < 4; ++st)
    k.v[st] = *reinterpret_cast<const bf16x8*>(kbuf + 32 * kh * ElemTraits<__bf16>::ROWB + ll.k[st]);
  return k;
}

DEV f32x16 score_from(const KFrag& k, const QFrag<__bf16>& qf) {
  f32x16 s = {};
#pragma unroll
  for (int st = 0; st < 4; ++st) s = mfma_bf16(k.v[st], qf.v[st], s);
  return s;
}

DEV VFrag load_vfrag(const char* vbuf, int kh, const LdsLanes& ll) {
  VFrag v;
#pragma unroll
  for (int sp = 0; sp < 2; ++sp)
#pragma unroll
    for (int dh = 0; dh < 2; ++dh) {
      const char* b = vbuf + (32 * kh + 16 * sp) * ElemTraits<__bf16>::ROWB;
      const s16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(b + ll.v[0][dh]));
      const s16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(b + ll.v[1][dh]));
      v.a[sp][dh] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(t0, t1, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  return v;
}

// Online-softmax update for one unit (bf16): returns the bf16 P operand.
DEV PFrag softmax_p(WaveAcc& acc, const f32x16& s, float c2) {
  float mx = s[0];
#pragma unroll
  for (int j = 1; j < 16; ++j) mx = fmaxf(mx, s[j]);
  if (__builtin_amdgcn_ballot_w64(mx > acc.thr)) {
    const float pm = pair_max(mx);
    const bool upd = pm > acc.thr;
    const float alpha = upd ? __builtin_amdgcn_exp2f((acc.m - pm) * c2) : 1.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) { acc.o[0][i] *= alpha; acc.o[1][i] *= alpha; }
    acc.l *= alpha;
    acc.m = upd ? pm : acc.m;
    acc.thr = acc.m + RESCALE_LOG2 / c2;
    acc.moff = acc.m == -__builtin_inff() ? 0.f : -acc.m * c2;
  }
  PFrag pf;
  float l = acc.l;
#pragma unroll
  for (int j = 0; j < 16; j += 2) {
    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j], c2, acc.moff));
    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j + 1], c2, acc.moff));
    const bf16x2 t = __builtin_convertvector(f32x2{p0, p1}, bf16x2);
    l += p0 + p1;
    pf.b[j >> 3][j & 7] = t[0];
    pf.b[j >> 3][(j & 7) + 1] = t[1];
  }
  acc.l = l;
  return pf;
}

// A band block's only global column (one global token for its batch item):
// the key enters the online-softmax state before the band, from registers.
// Each lane holds half of q and of k (d = 16s + 8g + e), so the score is the
// sum over the row's two lanes; against the reference m = that score its
// weight is exp2(0) = 1, so O starts as the key's V row (each lane its own
// d columns) and l as 1, counted on the row's first lane.
DEV void global_column_init(WaveAcc& acc, const QFrag<__bf16>& qf, const QFrag<__bf16>& kf,
                            const bf16x4 (&vr)[2][4], bool allowed, float c2, int g) {
  float part = 0.f;
#pragma unroll
  for (int st = 0; st < 4; ++st)
#pragma unroll
    for (int e = 0; e < 8; e += 2)
      part = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{qf.v[st][e], qf.v[st][e + 1]},
                                              bf16x2{kf.v[st][e], kf.v[st][e + 1]}, part, false);
  const float sc = pair_sum(part);
  if (allowed) {
    acc.m = sc;
    acc.thr = sc + RESCALE_LOG2 / c2;
    acc.moff = -sc * c2;
    acc.l = g == 0 ? 1.f : 0.f;
#pragma unroll
    for (int dh = 0; dh < 2; ++dh)
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc.o[dh][4 * a + e] = (float)vr[dh][a][e];
  }
}

DEV void pv_from(WaveAcc& acc, const VFrag& v, const PFrag& pf) {
#pragma unroll
  for (int sp = 0; sp < 2; ++sp)
#pragma unroll
    for (int dh = 0; dh < 2; ++dh) acc.o[dh] = mfma_bf16(v.a[sp][dh], pf.b[sp], acc.o[dh]);
}

// Mask one 32-key unit of a band tile: key kk = k0 + key_of_reg(j, g) is
// allowed for query qi iff qi - half <= kk <= min(qi + right, nr - 1).
template <class T>
DEV void mask_band_unit(f32x16& s, int k0, int qi, int half, int right, int nr, int g) {
  const int lo = qi - half - k0 - g * key_g_step<T>;
  const int hi = min(qi + right, nr - 1) - k0 - g * key_g_step<T>;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int off = key_reg_base<T>(j);
    if (off < lo || off > hi) s[j] = -__builtin_inff();
  }
}

// Store the normalised O rows owned by this lane (query row `pos`).
DEV void store_o(__bf16* orow, const WaveAcc& acc, float inv, int g) {
#pragma unroll
  for (int dh = 0; dh < 2; ++dh)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      bf16x4 t;
#pragma unroll
      for (int e = 0; e < 4; ++e) t[e] = (__bf16)(acc.o[dh][4 * a + e] * inv);
      *reinterpret_cast<bf16x4*>(orow + 32 * dh + 8 * a + 4 * g) = t;
    }
}
DEV void store_o(float* orow, const WaveAcc& acc, float inv, int g) {
#pragma unroll
  for (int dh = 0; dh < 2; ++dh)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      f32x4 t;
#pragma unroll
      for (int e = 0; e < 4; ++e) t[e] = acc.o[dh][4 * a + e] * inv;
      *reinterpret_cast<f32x4*>(orow + 32 * dh + 8 * a + 4 * g) = t;
    }
}

// Store a wave's 32 rows of 64 (an O, dQ, dK or dV accumulator, times `inv`,
// in bf16) so that every store instruction writes whole 128-byte rows, with
// non-temporal stores: the two lanes of row l put their halves into `slot` (4 KB of LDS that only this wave uses;
// 16-byte chunks permuted by the row's low bits against bank conflicts),
// then each lane reads back one 16-byte chunk of row 8k + lane/8 and stores
// it. Written this way the rows stream out past L2 instead of being left
// dirty for the write-back at the kernel's end. Row qw0 + i sits at
// position r + (qw0 + i) * dil; rows qw0 + i >= nr and position `skip` are
// skipped.
DEV void store_o_rows(char* slot, char* obase, const f32x16 (&o)[2], float inv, int lane, int qw0,
                      int nr, int r, int dil, int skip = -1) {
  typedef __attribute__((address_space(3))) char lds_char;
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  lds_char* s = (lds_char*)slot;
  const int l = lane & 31, g = lane >> 5;
#pragma unroll
  for (int dh = 0; dh < 2; ++dh)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      bf16x4 t;
#pragma unroll
      for (int e = 0; e < 4; ++e) t[e] = (__bf16)(o[dh][4 * a + e] * inv);
      const int pc = (4 * dh + a) ^ (l & 7);  // chunk 4dh+a holds d = 32dh+8a .. +7
      *reinterpret_cast<__attribute__((address_space(3))) bf16x4*>(s + l * 128 + pc * 16 + g * 8) = t;
    }
  // the same wave reads what it wrote: LDS keeps one wave's accesses in order
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int row = 8 * k + (lane >> 3), ch = lane & 7;
    const u32x4 v =
        *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(s + row * 128 + ((ch ^ (row & 7)) << 4));
    const int qi = qw0 + row;
    if (qi < nr && r + qi * dil != skip)
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(obase + (long)(r + qi * dil) * 128 + ch * 16));
  }
}

// ----------------------------------------------------------------------------
// Tile movement.

// Direct global->LDS load of one 64-row K tile and V tile (rows
// r + kk*dil, kk = kb0 .. kb0+63 clamped to kend-1) into `stage` (K at 0, V
// at KT*ROWB). Each wave issues PER_WAVE 1-KB instructions; lane l of an
// instruction lands at LDS byte 16*l of it, so it fetches the logical chunk
// that the swizzle places there.
template <class T>
struct Dma {
  static constexpr int ROWB = ElemTraits<T>::ROWB;
  static constexpr int CPR = ElemTraits<T>::CPR;
  static constexpr int RPI = 1024 / ROWB;            // rows per instruction
  static constexpr int NI = 2 * KT * ROWB / 1024;     // instructions per K+V tile
  static constexpr int PER_WAVE = NI / BAND_WAVES;    // per wave (bf16: 4, fp32: 8)
};

// One 16-byte-per-lane global->LDS load; `lds` is the wave-uniform LDS byte
// address of the 1-KB destination (held in M0). Written as a statement of its
// own so that the compiler does not track it as an LDS store: the band loop
// orders these loads against LDS reads itself (wait_vmcnt + wg_barrier). The
// instruction has no register result, so nothing is overwritten in flight.
DEV void dma16(const void* src, unsigned lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds)
               : "memory", "m0");
}

template <class T>
DEV void dma_tile(unsigned stage, const char* kb, const char* vb, int kb0, int kend, int r, int dil,
                  int wave, int lane) {
  using D = Dma<T>;
#pragma unroll
  for (int i = 0; i < D::PER_WAVE; ++i) {
    const int I = wave * D::PER_WAVE + i;  // wave-uniform
    const int tensor = I / (D::NI / 2);
    const int blk = I % (D::NI / 2);
    const int row = blk * D::RPI + lane / D::CPR;
    const int pc = lane % D::CPR;
    const int kk = min(kb0 + row, kend - 1);
    const char* src = (tensor ? vb : kb) + (long)(r + kk * dil) * D::ROWB +
                      (ElemTraits<T>::phys(row, pc) << 4);
    dma16(src, stage + (unsigned)(tensor * (KT * D::ROWB) + blk * 1024));
  }
}

// The same loads for a tile whose 64 rows all exist (kb0 + 63 < kend), with
// a wave-uniform 64-bit base in SGPRs and a loop-invariant 32-bit lane
// offset: address = kb|vb + (r + kb0*dil)*ROWB + blk*RPI*dil*ROWB + lane_off.
// The lane offset (row-within-block * dil * ROWB + swizzled chunk) depends
// only on the parity of the block (the swizzle reads bit 3 of the row), so
// two registers cover every instruction.
DEV void dma16_saddr(const char* base, unsigned off, unsigned lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds)
               : "memory", "m0");
}

template <class T>
struct DmaLanes {
  unsigned off[2];  // lane offset for even / odd blocks
};

template <class T>
DEV void dma_lanes_init(DmaLanes<T>& dl, int dil, int lane) {
  using D = Dma<T>;
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int row = par * D::RPI + lane / D::CPR;  // row within an even/odd block pair
    const int pc = lane % D::CPR;
    dl.off[par] = (unsigned)((lane / D::CPR) * dil * D::ROWB + (ElemTraits<T>::phys(row, pc) << 4));
  }
}

template <class T>
DEV void dma_tile_fast(unsigned stage, const DmaLanes<T>& dl, const char* kb, const char* vb,
                       int kb0, int r, int dil, int wave) {
  using D = Dma<T>;
  const long rowb = (long)(r + kb0 * dil) * D::ROWB;  // wave-uniform
#pragma unroll
  for (int i = 0; i < D::PER_WAVE; ++i) {
    const int I = wave * D::PER_WAVE + i;
    const int tensor = I / (D::NI / 2);
    const int blk = I % (D::NI / 2);
    const char* base = (tensor ? vb : kb) + rowb + (long)blk * D::RPI * dil * D::ROWB;
    dma16_saddr(base, dl.off[blk & 1], stage + (unsigned)(tensor * (KT * D::ROWB) + blk * 1024));
  }
}

// Register-staged tile movement (used by the global-column prologue and the
// global-row kernel).
template <class T, int NT>
struct TileRegs {
  static constexpr int NC = KT * ElemTraits<T>::CPR / NT;  // chunks per thread per tensor
  uint4 k[NC];
  uint4 v[NC];
};

template <class T, int NT>
DEV void tile_commit(const TileRegs<T, NT>& tr, char* klds, char* vlds, int tid) {
  constexpr int CPR = ElemTraits<T>::CPR;
#pragma unroll
  for (int u = 0; u < TileRegs<T, NT>::NC; ++u) {
    const int c = tid + NT * u;
    const int row = c / CPR, ch = c % CPR;
    const int off = ElemTraits<T>::lds_off(row, ch);
    *reinterpret_cast<uint4*>(klds + off) = tr.k[u];
    *reinterpret_cast<uint4*>(vlds + off) = tr.v[u];
  }
}

// ----------------------------------------------------------------------------
// The key-tile ring shared by band blocks and global-row blocks.

// Key side of a ring pass: tiles of 64 rows r + kk*dil, kk = kbeg + 64t,
// clamped to kend - 1, in LDS stages at a0/a1/a2.
struct RingCtx {
  unsigned a0, a1, a2;  // LDS byte addresses of the stages (a2 unused with 2)
  const char* kb;       // K rows of this (batch, head)
  const char* vb;       // V rows of this (batch, head)
  int kbeg, kend, nband, r, dil;
  int wave, lane, g;
  bool live;            // this wave has query rows to compute
  float c2;
  LdsLanes ll;          // lane offsets of the bf16 fragment reads
  int rot;              // the ring visits tiles rot, rot+1, .., nband-1, 0, .., rot-1
  bool fair;            // set wave priorities by the tiles left (band blocks)
};

// Tile index (0 .. nband-1) of ring step s.
DEV int ring_tile(const RingCtx& c, int s) {
  const int t = s + c.rot;
  return t < c.nband ? t : t - c.nband;
}

// Which 32-key units a band wave computes and how they are masked: row qi
// sees keys qi - half .. qi + right of its residue class, clipped to nr.
struct BandPol {
  int qi, qw0, half, right, nr, wk_lo, wk_hi;
  DEV bool active(int ku) const { return ku <= wk_hi && ku + 31 >= wk_lo; }
  DEV bool interior(int ku) const {
    return ku >= qw0 + 31 - half && ku + 31 <= qw0 + right && ku + 31 < nr;
  }
  template <class T> DEV void mask(f32x16& s, int ku, int g) const {
    mask_band_unit<T>(s, ku, qi, half, right, nr, g);
  }
};

// Global rows against a contiguous chunk of keys [.., k_hi): every key below
// k_hi, and left of the row when causal (lim = the row's position).
struct GlobPol {
  int lim, k_hi, gmin, causal;
  DEV bool active(int ku) const { return ku < k_hi; }
  DEV bool interior(int ku) const { return ku + 31 < k_hi && (!causal || ku + 31 <= gmin); }
  template <class T> DEV void mask(f32x16& s, int ku, int g) const {
    const int top = min(k_hi - 1, lim) - ku - g * key_g_step<T>;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (key_reg_base<T>(j) > top) s[j] = -__builtin_inff();
  }
};

// One step of the NS-stage ring (NS = 2 or 3) for tile tb, which sits in
// stage S: wait for it, publish it to the workgroup, start the DMA of tile
// tb+NS-1 into stage (S+NS-1)%NS (the stage of tile tb-1, which every wave
// has finished), and compute it. The stages are distinct LDS objects indexed
// statically, so the compiler can tell that the reads of stage S do not
// depend on the loads in flight to the others. Every step issues exactly one
// tile of DMA (past the last tile it re-fetches the last tile into a stage
// nobody reads again), so every step's wait has the same count.
template <class T, int NS, int S, class Pol>
DEV void ring_step(int tb, WaveAcc& acc, const QFrag<T>& qf, const RingCtx& c, const Pol& pol,
                   const DmaLanes<T>& dl, const char* st0, const char* st1, const char* st2) {
  constexpr int TILEB = KT * ElemTraits<T>::ROWB;
  const char* cur = S == 0 ? st0 : (S == 1 ? st1 : st2);
  constexpr int SN = (S + NS - 1) % NS;
  const unsigned nxt = SN == 0 ? c.a0 : (SN == 1 ? c.a1 : c.a2);
  if (c.fair) {
    // the workgroups sharing a CU otherwise run oldest-first, which leaves
    // the last one alone on the CU at the end; waves with more tiles left
    // issue first, so the co-resident workgroups finish together
    const int rem = c.nband - tb;
    if (rem >= 9) __builtin_amdgcn_s_setprio(3);
    else if (rem >= 6) __builtin_amdgcn_s_setprio(2);
    else if (rem >= 3) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
  }
  wait_vmcnt<NS == 3 ? Dma<T>::PER_WAVE : 0>();
  wg_barrier();  // tile tb has landed for every wave; tile tb-1 is consumed
  const int kn = c.kbeg + ring_tile(c, min(tb + NS - 1, c.nband - 1)) * KT;
  if (kn + KT <= c.kend) dma_tile_fast<T>(nxt, dl, c.kb, c.vb, kn, c.r, c.dil, c.wave);
  else dma_tile<T>(nxt, c.kb, c.vb, kn, c.kend, c.r, c.dil, c.wave, c.lane);
  if (!c.live) return;
  const int k0 = c.kbeg + ring_tile(c, tb) * KT;
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
    const int ku = k0 + 32 * kh;
    if (!pol.active(ku)) continue;  // wave-uniform skip
    if constexpr (sizeof(T) == 2) {
      f32x16 sc = score_from(load_kfrag(cur, kh, c.ll), qf);
      const VFrag v = load_vfrag(cur + TILEB, kh, c.ll);  // in flight during the softmax
      if (!pol.interior(ku)) pol.template mask<T>(sc, ku, c.g);
      pv_from(acc, v, softmax_p(acc, sc, c.c2));
    } else {
      f32x16 sc = score_unit(cur, kh, qf, c.lane);
      if (!pol.interior(ku)) pol.template mask<T>(sc, ku, c.g);
      softmax_pv_unit(acc, sc, cur + TILEB, kh, c.lane, c.c2);
    }
  }
}

// LDS ring depth and resulting waves per SIMD: bf16 tiles are 16 KB (K + V),
// so three stages (48 KB) leave room for three workgroups per CU; fp32 tiles
// are 32 KB.
template <class T> struct RingCfg;
template <> struct RingCfg<__bf16> { static constexpr int NS = 3; };
template <> struct RingCfg<float> { static constexpr int NS = 2; };

// Start the ring: DMA of tile 0 (and 1 with three stages).
template <class T>
DEV void ring_start(const RingCtx& c) {
  dma_tile<T>(c.a0, c.kb, c.vb, c.kbeg + ring_tile(c, 0) * KT, c.kend, c.r, c.dil, c.wave, c.lane);
  if (RingCfg<T>::NS == 3)
    dma_tile<T>(c.a1, c.kb, c.vb, c.kbeg + ring_tile(c, min(1, c.nband - 1)) * KT, c.kend, c.r, c.dil,
                c.wave, c.lane);
}

// Run every tile of the ring (ring_start has been issued and, with it, any
// earlier loads of this wave waited for).
template <class T, class Pol>
DEV void ring_run(WaveAcc& acc, const QFrag<T>& qf, const RingCtx& c, const Pol& pol,
                  const char* st0, const char* st1, const char* st2) {
  constexpr int NS = RingCfg<T>::NS;
  DmaLanes<T> dl;
  dma_lanes_init<T>(dl, c.dil, c.lane);
  for (int tb = 0; tb < c.nband; tb += NS) {
    ring_step<T, NS, 0>(tb, acc, qf, c, pol, dl, st0, st1, st2);
    if (tb + 1 < c.nband) ring_step<T, NS, 1>(tb + 1, acc, qf, c, pol, dl, st0, st1, st2);
    if (NS == 3 && tb + 2 < c.nband) ring_step<T, NS, NS - 1>(tb + 2, acc, qf, c, pol, dl, st0, st1, st2);
  }
  wait_vmcnt<0>();  // no load may still be writing LDS when the workgroup ends
}

// ----------------------------------------------------------------------------
// Band block: 128 query rows of one residue class, with the global columns
// folded in as extra key tiles.

typedef __attribute__((address_space(4))) const TileRec const_TileRec;

DEV TileRec decode_tile(const BandParams& p, int tile) {
  // the list is read-only for the whole launch: a scalar load
  TileRec t;
  if (p.tiles) {
    const_TileRec* x = (const_TileRec*)p.tiles + tile;
    t.bh = x->bh; t.r = x->r; t.q0 = x->q0; t.nr = x->nr;
    t.half = x->half; t.right = x->right; t.dil = x->dil; t.pad = 0;
    return t;
  }
  const int per_bh = p.uni_dil * p.uni_nqb;
  t.bh = tile / per_bh;
  const int rem = tile - t.bh * per_bh;
  t.r = rem / p.uni_nqb;
  t.q0 = (rem - t.r * p.uni_nqb) * BM;
  t.nr = (p.n - t.r + p.uni_dil - 1) / p.uni_dil;
  t.half = p.uni_half;
  t.right = p.uni_right;
  t.dil = p.uni_dil;
  t.pad = 0;
  return t;
}

// Global-column keys: the rows of the gather of keys t0 .. t0+63 that this
// lane's four load instructions fetch (clamped to the last global token).
DEV void gather_rows(int (&gq)[4], const int* gidx, int t0, int ng, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int blk = 4 * (wave & 1) + i;
    gq[i] = gidx[min(t0 + blk * Dma<__bf16>::RPI + lane / Dma<__bf16>::CPR, ng - 1)];
  }
}

// Direct global->LDS gather of K and V rows gq (absolute positions) into
// `stage`, laid out as a ring tile.
DEV void dma_gather(unsigned stage, const char* kb, const char* vb, const int (&gq)[4], int wave,
                    int lane) {
  using D = Dma<__bf16>;
  static_assert(D::PER_WAVE == 4, "four gather instructions per wave");
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int I = wave * 4 + i;
    const int tensor = I / (D::NI / 2);
    const int blk = I % (D::NI / 2);
    const int row = blk * D::RPI + lane / D::CPR;
    const char* src = (tensor ? vb : kb) + (long)gq[i] * D::ROWB +
                      (ElemTraits<__bf16>::phys(row, lane % D::CPR) << 4);
    dma16(src, stage + (unsigned)(tensor * (KT * D::ROWB) + blk * 1024));
  }
}

// Key metadata of a global-column tile: absolute position (or a value past
// every limit for padding) and residue-local index (or a sentinel when the
// key is not in this residue class).
DEV void gmeta_write(int (*gmeta)[KT], int kpos, bool real, int r, int dil, int tid) {
  int kp = 0x7fffffff, kr = NEG_SENTINEL;
  if (real) {
    kp = kpos;
    const int dr = kp - r;
    if (dr >= 0 && dr % dil == 0) kr = dr / dil;
  }
  gmeta[0][tid] = kp;
  gmeta[1][tid] = kr;
}

// The global-column units of one gathered tile (keys t0 ..): a key counts for
// row qi if it is left of the row when causal and not already in its band.
template <class T>
DEV void glob_cols_tile(WaveAcc& acc, const QFrag<T>& qf, const RingCtx& c, const char* stage,
                        const int (*gmeta)[KT], int t0, int ng, int qi, int half, int right, int lim) {
  constexpr int TILEB = KT * ElemTraits<T>::ROWB;
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
    if (t0 + 32 * kh >= ng) continue;
    f32x16 s;
    if constexpr (sizeof(T) == 2) s = score_from(load_kfrag(stage, kh, c.ll), qf);
    else s = score_unit(stage, kh, qf, c.lane);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int kk = 32 * kh + key_of_reg<T>(j, c.g);
      const int kp = gmeta[0][kk], kr = gmeta[1][kk];
      const bool inband = kr >= qi - half && kr <= qi + right;
      if (!(kp <= lim) || inband) s[j] = -__builtin_inff();
    }
    if constexpr (sizeof(T) == 2) pv_from(acc, load_vfrag(stage + TILEB, kh, c.ll), softmax_p(acc, s, c.c2));
    else softmax_pv_unit(acc, s, stage + TILEB, kh, c.lane, c.c2);
  }
}

// First ring step of a band block. Consecutive 128-row blocks of a residue
// class share most of their key tiles; blocks are taken in groups of
// (half + right + BM) / BM, about the number of blocks whose windows meet one
// key, and every block of a group starts at the tile that holds the middle of
// the group's middle block (clipped to its own band), then wraps around its
// band. At the start of the kernel, when every block fetches at once, a
// group then asks memory for one tile instead of one per block; the order of
// the tiles does not change the result.
DEV int band_rotation(int q0, int kbeg, int nband, int half, int right) {
  const int gs = max(1, (half + right + BM) / BM);
  const int qb = q0 / BM;
  const int anchor = (qb / gs * gs + gs / 2) * BM + BM / 2;
  const int t = anchor >= kbeg ? (anchor - kbeg) / KT : 0;
  return min(t, nband - 1);
}

// One 4-byte-per-lane global->LDS load (lane l lands at lds + 4 l).
DEV void dma4(const void* src, unsigned lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(lds)
               : "memory", "m0");
}

// Wait until this wave's LDS reads have returned (their registers are
// written), so that a barrier after it also orders them before later
// global->LDS loads into the same buffer.
DEV void wait_lgkm0() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xf | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
  asm volatile("" ::: "memory");
}

// A band block's 128 query rows (residue-local q0 .., clamped to nr - 1) of
// bf16 Q into a ring stage in the tiles' layout (row-major, 16-byte chunks
// swizzled): wave w loads its own 32 rows, eight per 1 KB load.
DEV void dma_qrows(unsigned stage, const char* qb, int q0, int nr, int r, int dil, int wave, int lane) {
  constexpr int ROWB = ElemTraits<__bf16>::ROWB;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 32 * wave + 8 * i + lane / 8;  // row of the block
    const int pc = lane % 8;                       // the chunk slot this lane fills
    const int kk = min(q0 + row, nr - 1);
    dma16(qb + (long)(r + kk * dil) * ROWB + (ElemTraits<__bf16>::phys(row, pc) << 4),
          stage + (unsigned)(1024 * (4 * wave + i)));
  }
}

template <class T>
DEV void band_block(const BandParams& p, int tile, int part, char* st0, char* st1, char* st2,
                    int (*gmeta)[KT]) {
  constexpr int ROWB = ElemTraits<T>::ROWB;
  constexpr int CPR = ElemTraits<T>::CPR;
  constexpr int TILEB = KT * ROWB;
  constexpr bool BF16 = sizeof(T) == 2;

  const int tid = threadIdx.x;
  const int lane = tid & 63, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // The indices of the first global-column tile go out right behind the
  // tile record's scalar load (with per-item sets, behind the set's offsets).
  const TileRec td = decode_tile(p, tile);
  const GSet gs = batch_gset(p.gidx, p.goff, p.ng, td.bh / p.H);
  const int* gix = gs.idx;
  const int ngb = part == 0 ? gs.n : 0;  // the global columns go with the first key part
  // with gskip (at most one global token per item) that token's row is the
  // global-row blocks' to write
  const int skip = p.gskip && gs.n > 0 ? gix[0] : -1;
  int gq[4] = {0, 0, 0, 0};
  int gm = 0;
  int gpos1 = 0;  // the global column when it is the only one (bf16)
  if (BF16 && ngb > 1) {
    gather_rows(gq, gix, 0, ngb, wave, lane);
    gm = gix[min(lane, ngb - 1)];
  } else if (BF16 && ngb == 1) {
    gpos1 = gix[0];
  }
  const int bh = td.bh, r = td.r, q0 = td.q0, nr = td.nr;
  if (q0 >= nr) return;  // an empty residue block (uniform decode only)
  const int half = td.half, right = td.right, dil = td.dil;
  const long base = (long)bh * p.n * ROWB;
  const char* kb = reinterpret_cast<const char*>(p.k) + base;
  const char* vb = reinterpret_cast<const char*>(p.v) + base;

  const int kbeg = max(0, q0 - half);
  const int kend = min(nr, q0 + BM + right);
  const int nband = (kend - kbeg + KT - 1) / KT;  // >= 1: row q0 sees itself
  // with a key split this workgroup takes band tiles t0 .. t1-1 (maybe none)
  const int t0 = part * nband / p.parts, t1 = (part + 1) * nband / p.parts;

  // this wave's query rows and key range (residue-local)
  const int qw0 = q0 + 32 * wave;
  const bool wave_live = qw0 < nr;
  const int qi = qw0 + (lane & 31);
  const bool row_ok = qi < nr;
  const int pos_q = r + min(qi, nr - 1) * dil;
  const int wk_lo = max(0, qw0 - half);
  const int wk_hi = min(nr - 1, qw0 + 31 + right);
  const int lim = p.causal ? pos_q : 0x7fffffff - 1;

  RingCtx c{(unsigned)(uintptr_t)(lds_void*)st0, (unsigned)(uintptr_t)(lds_void*)st1,
            (unsigned)(uintptr_t)(lds_void*)st2, kb, vb, kbeg + t0 * KT, kend, t1 - t0, r, dil,
            wave, lane, g, wave_live, p.c2, {}};
  lds_lanes_init(c.ll, lane);
  if (p.parts == 1) c.rot = band_rotation(q0, kbeg, c.nband, half, right);
  c.fair = p.fair != 0;
  const BandPol pol{qi, qw0, half, right, nr, wk_lo, wk_hi};
  const T* qrow = reinterpret_cast<const T*>(reinterpret_cast<const char*>(p.q) + base + (long)pos_q * ROWB);
  QFrag<T> qf;
  WaveAcc acc;
  acc_init(acc);

  if constexpr (BF16) {
   if (ngb <= 1) {
    // One round trip for what the block starts with, every load a direct
    // global->LDS one: the block's Q rows into stage 2 (free until ring step
    // 0 refills it), with one global token its K and V rows into the
    // global-column metadata's space (unused then), band tiles 0 and 1. The
    // block waits for all but tile 1, so that its first tile's compute runs
    // while tile 1 lands; Q and the global key then go to registers, and the
    // global column is folded in from there.
    QFrag<T> kgf;
    bf16x4 vgr[2][4];
    char* kgrow = reinterpret_cast<char*>(&gmeta[0][0]);  // K row (128 B), then V row
    dma_qrows(c.a2, reinterpret_cast<const char*>(p.q) + base, q0, nr, r, dil, wave, lane);
    if (ngb == 1 && wave == 0)
      dma4((lane < 32 ? kb : vb) + (long)gpos1 * ROWB + 4 * (lane & 31),
           (unsigned)(uintptr_t)(lds_void*)kgrow);
    if (c.nband > 0) {
      ring_start<T>(c);
      wait_vmcnt<Dma<T>::PER_WAVE>();  // everything but tile 1
    } else {
      wait_vmcnt<0>();
    }
    wg_barrier();  // every wave's rows of Q, the global key and tile 0 have landed
    {
      const int row = 32 * wave + (lane & 31);  // this lane's query row in the block
#pragma unroll
      for (int st = 0; st < 4; ++st)
        qf.v[st] = *reinterpret_cast<const bf16x8*>(st2 + ElemTraits<__bf16>::lds_off(row, 2 * st + g));
    }
    if (ngb == 1) {
#pragma unroll
      for (int st = 0; st < 4; ++st) kgf.v[st] = *reinterpret_cast<const bf16x8*>(kgrow + 16 * (2 * st + g));
#pragma unroll
      for (int dh = 0; dh < 2; ++dh)
#pragma unroll
        for (int a = 0; a < 4; ++a)
          vgr[dh][a] = *reinterpret_cast<const bf16x4*>(kgrow + ROWB + 2 * (32 * dh + 8 * a + 4 * g));
    }
    wait_lgkm0();  // the reads of stage 2 are done before ring step 0 refills it
    if (ngb == 1 && wave_live) {
      // the key counts for this row if it is left of the row when causal and
      // not already in the row's band
      const int dr = gpos1 - r;
      const bool same = dr >= 0 && dr % dil == 0;
      const bool inband = same && dr / dil >= qi - half && dr / dil <= qi + right;
      global_column_init(acc, qf, kgf, vgr, gpos1 <= lim && !inband, c.c2, g);
    }
   } else {
    // One round trip for everything the block starts with: the first
    // global-column tile into stage 2, band tiles 0 and 1 into stages 0 and
    // 1, and Q. (The gather goes first: the compiler waits for the indices
    // it needs with a count that only knows its own loads.)
    dma_gather(c.a2, kb, vb, gq, wave, lane);
    if (c.nband > 0) ring_start<T>(c);
    load_q(qf, qrow, g);
    if (ngb > 0) {
      if (tid < KT) gmeta_write(gmeta, gm, tid < ngb, r, dil, tid);
      wait_vmcnt<0>();
      __syncthreads();
      if (wave_live) glob_cols_tile<T>(acc, qf, c, st2, gmeta, 0, ngb, qi, half, right, lim);
      for (int t0 = KT; t0 < ngb; t0 += KT) {  // more than 64 global tokens
        gather_rows(gq, gix, t0, ngb, wave, lane);
        gm = gix[min(t0 + lane, ngb - 1)];
        __syncthreads();  // stage 2 and gmeta are free again
        dma_gather(c.a2, kb, vb, gq, wave, lane);
        if (tid < KT) gmeta_write(gmeta, gm, t0 + tid < ngb, r, dil, tid);
        wait_vmcnt<0>();
        __syncthreads();
        if (wave_live) glob_cols_tile<T>(acc, qf, c, st2, gmeta, t0, ngb, qi, half, right, lim);
      }
      // the first ring step's barrier orders these reads of stage 2 before
      // the load of band tile 2 into it
    }
   }
  } else {
    // fp32: two ring stages; the global columns go through stage 0 first
    load_q(qf, qrow, g);
    wait_vmcnt<0>();
    if (ngb > 0) {
      constexpr int NC = TileRegs<T, 256>::NC;
      for (int t0 = 0; t0 < ngb; t0 += KT) {
        TileRegs<T, 256> tr;
        int gp[NC];
#pragma unroll
        for (int u = 0; u < NC; ++u) gp[u] = gix[min(t0 + (tid + 256 * u) / CPR, ngb - 1)];
#pragma unroll
        for (int u = 0; u < NC; ++u) {
          const long off = (long)gp[u] * ROWB + ((tid + 256 * u) % CPR) * 16;
          tr.k[u] = *reinterpret_cast<const uint4*>(kb + off);
          tr.v[u] = *reinterpret_cast<const uint4*>(vb + off);
        }
        if (tid < KT) gmeta_write(gmeta, gix[min(t0 + tid, ngb - 1)], t0 + tid < ngb, r, dil, tid);
        tile_commit<T, 256>(tr, st0, st0 + TILEB, tid);
        __syncthreads();
        if (wave_live) glob_cols_tile<T>(acc, qf, c, st0, gmeta, t0, ngb, qi, half, right, lim);
        __syncthreads();
      }
    }
    if (c.nband > 0) ring_start<T>(c);
  }

  // band tiles through the ring: the loads of the next tiles are in flight
  // while tile t is computed. Rows past the band end are clamped to a valid
  // row; their scores are masked, so their values only ever meet p = 0.
  ring_run<T>(acc, qf, c, pol, st0, st1, st2);

  if (wave_live) {
    const float ltot = pair_sum(acc.l);
    if (row_ok && p.parts > 1) {
      // unnormalised partial for band_merge (m = -inf, l = 0 without keys)
      float* rec = p.part + (((long)bh * p.n + pos_q) * p.parts + part) * PART_STRIDE;
      store_o(rec, acc, 1.0f, g);
      if (g == 0) *reinterpret_cast<f32x2*>(rec + HD) = f32x2{acc.m, ltot};
    } else if (BF16 && c.nband > 0) {
      // The stage of ring step nband takes the rows: nobody reads it again,
      // and every wave's loads into it completed before the last ring
      // barrier (issued at step nband-2, or by ring_start when nband = 1,
      // and waited for at step nband-1 or before the ring). Each wave uses
      // the 4 KB at 4096 * wave.
      const int sa = c.nband % 3;
      char* slot = (sa == 0 ? st0 : (sa == 1 ? st1 : st2)) + 4096 * wave;
      store_o_rows(slot, reinterpret_cast<char*>(p.o) + base, acc.o, 1.0f / ltot, lane, qw0, nr, r, dil, skip);
      if (row_ok && pos_q != skip && p.lse && g == 0) p.lse[(long)bh * p.n + pos_q] = acc.m * p.scale + __logf(ltot);
    } else if (row_ok && pos_q != skip) {
      const float inv = 1.0f / ltot;
      T* orow = reinterpret_cast<T*>(reinterpret_cast<char*>(p.o) + base + (long)pos_q * ROWB);
      store_o(orow, acc, inv, g);
      if (p.lse && g == 0) p.lse[(long)bh * p.n + pos_q] = acc.m * p.scale + __logf(ltot);
    }
  }
}

// ----------------------------------------------------------------------------
// Global-row block: up to 4 x 32 global rows (one block of 32 per wave)
// against one chunk of keys of Kg, Vg; writes an unnormalised partial
// (o, m, l) per row and chunk. Block index = split + nsplit*(group +
// ngroup*bh).

template <class T>
DEV void global_block(const GlobalParams& p, int gb, char* st0, char* st1, char* st2) {
  constexpr int ROWB = ElemTraits<T>::ROWB;
  const int tid = threadIdx.x;
  const int lane = tid & 63, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sp = gb % p.nsplit;
  const int grp = (gb / p.nsplit) % p.ngroup;
  const int bh = gb / (p.nsplit * p.ngroup);
  const long base = (long)bh * p.n * ROWB;
  const GSet gs = batch_gset(p.gidx, p.goff, p.ng, bh / p.H);
  if (gs.n <= grp * BAND_WAVES * 32) return;  // no rows of this item's set in this group

  const int qb = grp * BAND_WAVES + wave;  // this wave's block of 32 global rows
  const bool live = qb * 32 < gs.n;
  const int gi = qb * 32 + (lane & 31);
  const int pos_q = gs.idx[min(gi, gs.n - 1)];
  // G is sorted: the first row of the wave and the last row of the group
  // bound the causal key ranges.
  const int gmin = gs.idx[min(qb * 32, gs.n - 1)];
  const int gmax = gs.idx[min(grp * BAND_WAVES * 32 + BAND_WAVES * 32 - 1, gs.n - 1)];
  const int k_lo = sp * p.ksplit;
  int k_hi = min(p.n, k_lo + p.ksplit);
  if (p.causal) k_hi = min(k_hi, gmax + 1);
  const int nband = k_hi > k_lo ? (k_hi - k_lo + KT - 1) / KT : 0;  // workgroup-uniform

  RingCtx c{(unsigned)(uintptr_t)(lds_void*)st0, (unsigned)(uintptr_t)(lds_void*)st1,
            (unsigned)(uintptr_t)(lds_void*)st2,
            reinterpret_cast<const char*>(p.kg) + base, reinterpret_cast<const char*>(p.vg) + base,
            k_lo, k_hi, nband, 0, 1, wave, lane, g, live, p.c2, {}};
  lds_lanes_init(c.ll, lane);
  const GlobPol pol{p.causal ? pos_q : 0x7fffffff - 1, k_hi, gmin, p.causal};
  QFrag<T> qf;
  WaveAcc acc;
  acc_init(acc);
  if (nband > 0) {
    ring_start<T>(c);
    load_q(qf, reinterpret_cast<const T*>(reinterpret_cast<const char*>(p.qg) + base + (long)pos_q * ROWB), g);
    wait_vmcnt<0>();
    ring_run<T>(acc, qf, c, pol, st0, st1, st2);
  }

  if (live) {
    const float ltot = pair_sum(acc.l);
    if (gi < gs.n) {
      const long slot = ((long)bh * p.ng + gi) * p.nsplit + sp;
      float* po = p.part_o + slot * HD;
#pragma unroll
      for (int dh = 0; dh < 2; ++dh)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          f32x4 t;
#pragma unroll
          for (int e = 0; e < 4; ++e) t[e] = acc.o[dh][4 * a + e];
          *reinterpret_cast<f32x4*>(po + 32 * dh + 8 * a + 4 * g) = t;
        }
      if (g == 0) {
        p.part_ml[slot * 2 + 0] = acc.m;
        p.part_ml[slot * 2 + 1] = ltot;
      }
    }
  }
}

// Fold a partial (m, l, a) of one output column into a running (M, L, A):
// maxima in raw score units, weights exp2((score - max) * c2).
DEV void lse_fold(float& M, float& L, float& A, float m, float l, float a, float c2) {
  const float mn = fmaxf(M, m);
  const float fo = M == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f((M - mn) * c2);
  const float fn = m == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f((m - mn) * c2);
  L = L * fo + l * fn;
  A = A * fo + a * fn;
  M = mn;
}

// Rounds of 16 keys each wave of a streaming global-row block keeps in
// flight (8 would be a whole 512-key chunk, but spill registers at three
// waves per SIMD).
constexpr int GSTREAM_DEPTH = 6;

// ----------------------------------------------------------------------------
// Global row by streaming, for bf16 plans with at most one global token per
// batch item (a classification token): the row's keys are cut into chunks
// and block (bh, split) streams one chunk of Kg, Vg straight into registers.
// Four lanes hold a key (lane % 4 holds features 16 (lane % 4) .. +15): the
// score is eight fp32 dot products of bf16 pairs plus the other lanes'
// parts; each lane runs its own online softmax over its keys (the lazily
// raised reference max of the band path) and accumulates P V for its 16
// features in fp32. The matrix cores would compute 32 rows for the one that
// exists; what bounds this work is the stream of Kg and Vg: with 16 features
// per lane a lane's registers hold GSTREAM_DEPTH rounds of 16 keys per wave,
// most of a 512-key chunk, in flight at once. The block then folds its
// lanes' partial sums through LDS into one (o, m, l) record per chunk, the
// record global_block writes.
template <class T>
DEV void global_row_stream(const GlobalParams& p, int gb, char* st0, char* st1, char* st2) {
  if constexpr (sizeof(T) != 2) {
    return;  // the host streams bf16 plans only
  } else {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) char lds_char;
    constexpr int LPK = 4;              // lanes per key
    constexpr int DPL = HD / LPK;       // features per lane
    constexpr int CH = DPL * 2 / 16;    // 16-byte pieces of a lane's features
    constexpr int KPW = 64 / LPK;       // keys per wave and round
    constexpr int DEPTH = GSTREAM_DEPTH;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int sp = gb % p.nsplit, bh = gb / p.nsplit;
    const int k_lo = sp * p.ksplit;
    const int k_end = min(p.n, k_lo + p.ksplit);  // the chunk (k_lo < k_end)
    const long base = (long)bh * p.n * 128;
    const int part = lane % LPK, kq = lane / LPK;
    const char* kb = reinterpret_cast<const char*>(p.kg) + base + part * (2 * DPL);
    const char* vb = reinterpret_cast<const char*>(p.vg) + base + part * (2 * DPL);

    // round it, wave w: keys k_lo + KPW (4 it + w) + kq (clamped to the
    // chunk for the loads, which the first DEPTH rounds issue before the
    // global token's position is known)
    auto key = [&](int it) { return k_lo + KPW * (4 * it + wave) + kq; };
    auto fetch = [&](int it, u32x4 (&kk)[CH], u32x4 (&vv)[CH]) {
      const long j = min(key(it), k_end - 1);
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        kk[c] = *reinterpret_cast<const u32x4*>(kb + j * 128 + 16 * c);
        vv[c] = *reinterpret_cast<const u32x4*>(vb + j * 128 + 16 * c);
      }
    };
    const int nit_ld = (k_end - k_lo + 4 * KPW - 1) / (4 * KPW);
    u32x4 kbuf[DEPTH][CH], vbuf[DEPTH][CH];
#pragma unroll
    for (int s = 0; s < DEPTH; ++s)
      if (s < nit_ld) fetch(s, kbuf[s], vbuf[s]);
    const GSet gs = batch_gset(p.gidx, p.goff, p.ng, bh / p.H);
    if (gs.n == 0) return;  // workgroup-uniform: no global row in this item
    const int pos = gs.idx[0];
    const int k_hi = p.causal ? min(k_end, pos + 1) : k_end;
    const int nit = k_hi > k_lo ? (k_hi - k_lo + 4 * KPW - 1) / (4 * KPW) : 0;  // 4 KPW keys per round
    u32x4 q[CH];
    const char* qrow = reinterpret_cast<const char*>(p.qg) + base + (long)pos * 128 + part * (2 * DPL);
#pragma unroll
    for (int c = 0; c < CH; ++c) q[c] = *reinterpret_cast<const u32x4*>(qrow + 16 * c);

    float o[DPL];
#pragma unroll
    for (int i = 0; i < DPL; ++i) o[i] = 0.f;
    float m = -__builtin_inff(), thr = -__builtin_inff(), moff = 0.f, l = 0.f;
    auto bf2 = [](unsigned u) { return __builtin_bit_cast(bf16x2, u); };
    auto step = [&](int it, const u32x4 (&kk)[CH], const u32x4 (&vv)[CH]) {
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) s = __builtin_amdgcn_fdot2_f32_bf16(bf2(q[c][e]), bf2(kk[c][e]), s, false);
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      if (key(it) >= k_hi) s = -__builtin_inff();
      if (s > thr) {  // the same decision on the lanes of a key
        const float f = __builtin_amdgcn_exp2f((m - s) * p.c2);  // 0 while m = -inf
#pragma unroll
        for (int i = 0; i < DPL; ++i) o[i] *= f;
        l *= f;
        m = s;
        thr = s + RESCALE_LOG2 / p.c2;
        moff = -s * p.c2;
      }
      const float w = __builtin_amdgcn_exp2f(__builtin_fmaf(s, p.c2, moff));  // 0 for s = -inf
      l += w;
#pragma unroll
      for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const unsigned u = vv[c][e];
          o[8 * c + 2 * e] = __builtin_fmaf(w, __builtin_bit_cast(float, u << 16), o[8 * c + 2 * e]);
          o[8 * c + 2 * e + 1] = __builtin_fmaf(w, __builtin_bit_cast(float, u & 0xffff0000u), o[8 * c + 2 * e + 1]);
        }
    };
    for (int it0 = 0; it0 < nit; it0 += DEPTH) {
#pragma unroll
      for (int s = 0; s < DEPTH; ++s) {
        const int it = it0 + s;
        if (it < nit) {
          step(it, kbuf[s], vbuf[s]);
          if (it + DEPTH < nit) fetch(it + DEPTH, kbuf[s], vbuf[s]);
        }
      }
    }

    // fold: block max, each lane's sums scaled to it, then summed over the
    // KPW keys of a wave (LDS rows of 64 features, 16-byte chunks swizzled
    // by the key) and over the four waves
    typedef __attribute__((address_space(3))) float lds_float;
    lds_float* sm = (lds_float*)(lds_char*)st2;  // [4] maxima, [4] sums, then [4][64] wave sums
    float wm = m;
#pragma unroll
    for (int x = 1; x < 64; x <<= 1) wm = fmaxf(wm, __shfl_xor(wm, x));
    if (lane == 0) sm[wave] = wm;
    __syncthreads();
    const float M = fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
    const float f = m == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f((m - M) * p.c2);
    float lw = l * f;  // the lanes of a key hold the same l
#pragma unroll
    for (int x = LPK; x < 64; x <<= 1) lw += __shfl_xor(lw, x);
    lds_char* wb = (lds_char*)(st0 + 4096 * wave);  // [KPW][64] floats
#pragma unroll
    for (int c = 0; c < DPL / 4; ++c) {
      f32x4 t;
#pragma unroll
      for (int e = 0; e < 4; ++e) t[e] = o[4 * c + e] * f;
      *reinterpret_cast<__attribute__((address_space(3))) f32x4*>(wb + kq * 256 + part * (4 * DPL) +
                                                                   16 * (c ^ (kq % (DPL / 4)))) = t;
    }
    if (lane == 0) sm[4 + wave] = lw;
    __syncthreads();
    {
      const int d = lane, pd = d / DPL, c = (d % DPL) / 4;
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < KPW; ++k)
        acc += *reinterpret_cast<const __attribute__((address_space(3))) float*>(
            wb + k * 256 + pd * (4 * DPL) + 16 * (c ^ (k % (DPL / 4))) + 4 * (d % 4));
      sm[8 + 64 * wave + d] = acc;
    }
    __syncthreads();
    if (wave != 0) return;
    const int d = lane;
    const float od = sm[8 + d] + sm[8 + 64 + d] + sm[8 + 128 + d] + sm[8 + 192 + d];
    const float L = sm[4] + sm[5] + sm[6] + sm[7];
    const long row0 = ((long)bh * p.ng + 0) * p.nsplit;  // the item's one global row, gi = 0
    if (!p.fuse) {  // global_rows_merge folds the chunks after the kernel
      p.part_o[(row0 + sp) * HD + d] = od;
      if (d == 0) *reinterpret_cast<f32x2*>(p.part_ml + (row0 + sp) * 2) = f32x2{M, L};
      return;
    }
    // The chunks' last block folds them. The records move only through
    // device-scope atomic stores and loads, which bypass the XCDs' separate
    // L2 caches; a block's stores are complete (vmcnt 0) before its arrival
    // on the (batch, head) counter, and the last arrival (the counter's old
    // value nsplit - 1) issues its loads after the count has returned, so it
    // reads every record. No cache-wide write-back or invalidate is needed,
    // and the band blocks around keep their L2 contents. The last arrival
    // resets the counter for the next launch; band blocks leave the row alone.
    __hip_atomic_store(p.part_o + (row0 + sp) * HD + d, od, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (d == 0) {
      __hip_atomic_store(p.part_ml + (row0 + sp) * 2, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(p.part_ml + (row0 + sp) * 2 + 1, L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    wait_vmcnt<0>();
    int old = 0;
    if (d == 0) old = __hip_atomic_fetch_add(p.gcount + bh, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __shfl(old, 0);
    if (old != p.nsplit - 1) return;  // wave-uniform
    if (d == 0) __hip_atomic_store(p.gcount + bh, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    float FM = -__builtin_inff(), FL = 0.f, FA = 0.f;
    for (int b0 = 0; b0 < p.nsplit; b0 += 8) {
      float mm[8], ll[8], oo[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const long si = row0 + min(b0 + i, p.nsplit - 1);
        mm[i] = __hip_atomic_load(p.part_ml + si * 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ll[i] = __hip_atomic_load(p.part_ml + si * 2 + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        oo[i] = __hip_atomic_load(p.part_o + si * HD + d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (b0 + i < p.nsplit) lse_fold(FM, FL, FA, mm[i], ll[i], oo[i], p.c2);
    }
    // the row attends at least to its own key, so FL > 0
    T* orow = reinterpret_cast<T*>(p.o) + ((long)bh * p.n + pos) * HD;
    orow[d] = (T)(FA / FL);
    if (p.lse && d == 0) p.lse[(long)bh * p.n + pos] = FM * p.scale + __logf(FL);
  }
}

// ----------------------------------------------------------------------------
// The forward kernel: blocks [0, nband_blocks) are band blocks, the rest
// global-row blocks. The band blocks come first so that all of them start in
// the first wave of workgroups; the short global-row blocks fill the
// workgroup slots that band blocks at the sequence ends free early.

// GSTREAM: the instantiation for plans whose global rows are streamed
// (global_row_stream); the others leave that code out of their kernel.
template <class T, bool GSTREAM>
__global__ __launch_bounds__(256, 3) void attn_fwd(BandParams bp, GlobalParams gp, int nband_blocks) {
  constexpr int STAGEB = 2 * KT * ElemTraits<T>::ROWB;
  constexpr int NS = RingCfg<T>::NS;
  __shared__ __attribute__((aligned(1024))) char st0[STAGEB];
  __shared__ __attribute__((aligned(1024))) char st1[STAGEB];
  __shared__ __attribute__((aligned(1024))) char st2[NS == 3 ? STAGEB : 1024];
  __shared__ int gmeta[2][KT];  // global-column tile: key position, residue-local index
  const int b = blockIdx.x;
  if (b < nband_blocks) {
    // the key parts of one tile are adjacent, so they share an XCD's L2
    const int lb = xcd_remap(b, nband_blocks);
    band_block<T>(bp, lb / bp.parts, lb % bp.parts, st0, st1, st2, gmeta);
  }
  else if constexpr (GSTREAM) global_row_stream<T>(gp, b - nband_blocks, st0, st1, st2);
  else global_block<T>(gp, b - nband_blocks, st0, st1, st2);
}

// Merge of the key parts of every row (with a key split): 16 rows per
// 256-thread block, 16 threads per row, each owning 4 output columns. All
// parts of a row are loaded at once, then folded by their maxima as in the
// online softmax; every row has at least its own key, so the total weight is
// positive.
DEV void store4(__bf16* dst, f32x4 v) {
  bf16x4 t;
#pragma unroll
  for (int e = 0; e < 4; ++e) t[e] = (__bf16)v[e];
  *reinterpret_cast<bf16x4*>(dst) = t;
}
DEV void store4(float* dst, f32x4 v) { *reinterpret_cast<f32x4*>(dst) = v; }

template <class T>
__global__ __launch_bounds__(256) void band_merge(BandParams p, long rows) {
  const long row = (long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int c4 = (threadIdx.x & 15) * 4;
  if (row >= rows) return;
  const float* rec = p.part + row * p.parts * PART_STRIDE;
  f32x2 ml[MAX_KEY_SPLIT];
  f32x4 o[MAX_KEY_SPLIT];
#pragma unroll
  for (int k = 0; k < MAX_KEY_SPLIT; ++k)
    if (k < p.parts) {
      ml[k] = *reinterpret_cast<const f32x2*>(rec + k * PART_STRIDE + HD);
      o[k] = *reinterpret_cast<const f32x4*>(rec + k * PART_STRIDE + c4);
    }
  float M = -__builtin_inff();
#pragma unroll
  for (int k = 0; k < MAX_KEY_SPLIT; ++k)
    if (k < p.parts) M = fmaxf(M, ml[k][0]);
  float L = 0.f;
  f32x4 A = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < MAX_KEY_SPLIT; ++k)
    if (k < p.parts) {
      // a part with no key of this row has m = -inf, l = 0, o = 0
      const float f = ml[k][0] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f((ml[k][0] - M) * p.c2);
      L += ml[k][1] * f;
#pragma unroll
      for (int e = 0; e < 4; ++e) A[e] += o[k][e] * f;
    }
  const float inv = 1.0f / L;
#pragma unroll
  for (int e = 0; e < 4; ++e) A[e] *= inv;
  store4(reinterpret_cast<T*>(p.o) + row * HD + c4, A);
  if (p.lse && c4 == 0) p.lse[row] = M * p.scale + __logf(L);
}

constexpr int MAX_SPLIT = 256;

// Log-sum-exp merge of the key chunks of the global rows; overwrites rows G
// of O (and LSE). One wave per (b*h, global row), four rows per 256-thread
// block, so that every wave of the grid is resident at once and the merge is
// one memory round trip: lane d owns output column d and issues the loads of
// up to 16 chunks' column d together with their (max, sum) records, which
// are the same for every lane of the wave (scalar loads); the batch is folded
// against its own maximum, and batches (rows of more than 16 chunks) into a
// running (max, sum, output).
//
// The partials' pointers come first among the arguments so that they are
// preloaded into SGPRs (the build's kernarg-preload count) and the loads go
// out as the waves start.
template <class T>
__global__ __launch_bounds__(256) void global_rows_merge(const float* part_ml, const float* part_o,
                                                         int ng, int nsplit, int nrows, GlobalParams p) {
  constexpr int NB = 16;  // chunks per batch
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), d = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + wave;  // bh * ng + gi
  if (row >= nrows) return;                // wave-uniform
  const int bh = row / ng, gi = row - bh * ng;
  const GSet gs = batch_gset(p.gidx, p.goff, ng, bh / p.H);
  if (gi >= gs.n) return;  // not a row of this item's set
  const float* ml = part_ml + (long)row * nsplit * 2;
  const float* po = part_o + (long)row * nsplit * HD + d;
  float M = -__builtin_inff(), L = 0.f, A = 0.f;
  for (int s0 = 0; s0 < nsplit; s0 += NB) {
    float m[NB], l[NB], o[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const bool ok = s0 + i < nsplit;  // wave-uniform
      m[i] = ok ? ml[2 * (s0 + i)] : -__builtin_inff();
      l[i] = ok ? ml[2 * (s0 + i) + 1] : 0.f;
      o[i] = ok ? po[(long)(s0 + i) * HD] : 0.f;
    }
    float mb = M;
#pragma unroll
    for (int i = 0; i < NB; ++i) mb = fmaxf(mb, m[i]);
    // every chunk and the running state against the batch maximum (weights
    // 0 for empty chunks, m = -inf; mb stays -inf only if everything so far
    // is empty, and then L and A are 0)
    const float fr = M == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f((M - mb) * p.c2);
    L *= fr;
    A *= fr;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const float w = m[i] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f((m[i] - mb) * p.c2);
      L = __builtin_fmaf(l[i], w, L);
      A = __builtin_fmaf(o[i], w, A);
    }
    M = mb;
  }
  // the row attends at least to its own key, so L > 0
  const int pos = gs.idx[gi];
  T* orow = reinterpret_cast<T*>(p.o) + ((long)bh * p.n + pos) * HD;
  orow[d] = (T)(A / L);
  if (p.lse && d == 0) p.lse[(long)bh * p.n + pos] = M * p.scale + __logf(L);
}

}  // namespace swattn
