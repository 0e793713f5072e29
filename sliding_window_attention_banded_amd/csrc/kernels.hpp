// Device kernels of the banded sliding-window attention forward pass (gfx950).
//
// Operation (Longformer summary page, section 3-1 "Attention Pattern", and
// section 7 for the left-only mask): row i of head h attends to the keys
// i + k*dil_h, k in [-w_h/2, R_h] (R_h = 0 when causal, else w_h/2), plus
// every global token (left of i when causal), each key once; rows of the
// global tokens attend to every key through the separate projections Qg, Kg,
// Vg. Softmax scale 1/sqrt(64).
//
// Work decomposition (all three kernels share the wave-level tile engine):
//  * band_fwd: one workgroup = 4 waves = 128 query rows of one residue class
//    r (rows r, r+dil, r+2*dil, ... of one (batch, head)); within a residue
//    class the dilated window is an ordinary window of w+1 keys, so K/V rows
//    are read with a row stride of dil*64 elements and no key is wasted on
//    the gaps. Key tiles of 64 rows are double-buffered in LDS and shared by
//    the 4 waves; each wave skips the 32-key halves that lie outside its own
//    32 rows' band. The global columns are extra key tiles gathered from
//    K[G], V[G], masked so that a global key already inside the band is not
//    counted twice; the running max/sum of the online softmax merges them
//    with the band exactly as a log-sum-exp merge would.
//  * global_rows_partial: rows of G against a chunk of all keys with Qg, Kg,
//    Vg; writes an unnormalised partial (o, m, l) per chunk.
//  * global_rows_merge: log-sum-exp merge of the chunks; overwrites rows G of
//    O (and LSE), stream-ordered after band_fwd.
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
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

#define DEV __device__ __forceinline__

constexpr int HD = 64;        // head dimension
constexpr int KT = 64;        // keys per LDS tile
constexpr int BAND_WAVES = 4; // waves per band workgroup
constexpr int BM = 32 * BAND_WAVES;  // query rows per band workgroup
constexpr int NEG_SENTINEL = -(1 << 30);
constexpr float LOG2E = 1.4426950408889634f;

struct HeadInfo {
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
  const int4* tiles;     // {b*H + h, residue r, first residue-local row, 0}
  const HeadInfo* heads; // [H]
  const int* gidx;       // sorted G, [ng]
  int ng;
  int H;
  int n;
  int causal;
  float c2;     // scale * log2(e)
  float scale;  // 1/sqrt(64)
};

struct GlobalParams {
  const void* qg;
  const void* kg;
  const void* vg;
  void* o;
  float* lse;
  const int* gidx;
  float* part_o;  // [BH][ng][nsplit][64]
  float* part_ml; // [BH][ng][nsplit][2]  (max, sum)
  int ng;
  int n;
  int causal;
  int nsplit;
  int ksplit;   // keys per split, multiple of 64
  int nqb;      // ceil(ng / 32)
  float c2;
  float scale;
};

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

// MFMA row r of the S^T tile -> key within the 32-key half (swap bits 2, 3).
DEV int kperm16(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }
// fp32 variant: MFMA row r = 8a + 4g + b -> key 8a + 2b + g.
DEV int kperm32(int r) { return (r & ~7) | ((r & 3) << 1) | ((r >> 2) & 1); }

// key (within the 32-key half) held by accumulator register j of lane group g
DEV int key_of_reg16(int j, int g) { return ((j >> 3) << 4) + (g << 3) + (j & 7); }
DEV int key_of_reg32(int j, int g) { return 2 * j + g; }

DEV f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
DEV f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

DEV float wave_xor32(float x) { return __shfl_xor(x, 32, 64); }

template <class T> struct ElemTraits;
template <> struct ElemTraits<__bf16> {
  static constexpr int ROWB = 128;           // bytes per K/V row
  static constexpr int CPR = ROWB / 16;      // 16-byte chunks per row
  static DEV int lds_off(int row, int ch) { return row * ROWB + ((ch ^ swz(row)) << 4); }
};
template <> struct ElemTraits<float> {
  static constexpr int ROWB = 256;
  static constexpr int CPR = ROWB / 16;
  static DEV int lds_off(int row, int ch) { return row * ROWB + (ch << 4); }
};

// ----------------------------------------------------------------------------
// Wave-level tile engine.
//
// State of one wave: 32 query rows (one per lane pair l, l+32), running max m
// (raw score units), this lane's partial sum l, and O^T accumulators for the
// two 32-wide halves of d.
template <class T> struct QFrag;
template <> struct QFrag<__bf16> { bf16x8 v[4]; };  // d = 16s + 8g + e
template <> struct QFrag<float> { float v[32]; };   // d = 2s + g

struct WaveAcc {
  f32x16 o[2];
  float m;
  float l;
};

DEV void acc_init(WaveAcc& a) {
  for (int i = 0; i < 16; ++i) { a.o[0][i] = 0.f; a.o[1][i] = 0.f; }
  a.m = -__builtin_inff();
  a.l = 0.f;
}

// Load the B operand of S^T = K Q^T for this lane's query row (global memory).
DEV void load_q(QFrag<__bf16>& qf, const __bf16* row, int g) {
  const uint4* p = reinterpret_cast<const uint4*>(row);
  for (int s = 0; s < 4; ++s) qf.v[s] = __builtin_bit_cast(bf16x8, p[2 * s + g]);
}
DEV void load_q(QFrag<float>& qf, const float* row, int g) {
  for (int s = 0; s < 32; ++s) qf.v[s] = row[2 * s + g];
}

// S^T for one 32-key half of the LDS tile: 16 fp32 values per lane.
DEV f32x16 score_half(const char* kbuf, int kh, const QFrag<__bf16>& qf, int lane) {
  const int g = lane >> 5;
  const int row = kperm16(lane & 31) + 32 * kh;
  f32x16 s;
  for (int i = 0; i < 16; ++i) s[i] = 0.f;
  for (int st = 0; st < 4; ++st) {
    bf16x8 a = *reinterpret_cast<const bf16x8*>(kbuf + ElemTraits<__bf16>::lds_off(row, 2 * st + g));
    s = mfma_bf16(a, qf.v[st], s);
  }
  return s;
}
DEV f32x16 score_half(const char* kbuf, int kh, const QFrag<float>& qf, int lane) {
  const int g = lane >> 5;
  const int row = kperm32(lane & 31) + 32 * kh;
  const float* kr = reinterpret_cast<const float*>(kbuf + row * ElemTraits<float>::ROWB);
  f32x16 s;
  for (int i = 0; i < 16; ++i) s[i] = 0.f;
  for (int st = 0; st < 32; ++st) s = mfma_f32(kr[2 * st + g], qf.v[st], s);
  return s;
}

// O^T += V^T P^T for one 32-key half whose probabilities are p (accumulator
// layout of score_half).
DEV void pv_half(WaveAcc& acc, const char* vbuf, int kh, const f32x16& p, int lane) {
  const int g = lane >> 5;
  const int i16 = lane & 15;
  for (int sp = 0; sp < 2; ++sp) {
    bf16x8 b;
    for (int e = 0; e < 8; ++e) b[e] = (__bf16)p[8 * sp + e];
    for (int dh = 0; dh < 2; ++dh) {
      const int d0 = 32 * dh + 16 * ((lane >> 4) & 1);
      bf16x8 a;
      for (int hx = 0; hx < 2; ++hx) {
        // source lane (as a 16-lane group member) points at 4 d-contiguous
        // elements of key key0 + i16/4, columns d0 + 4*(i16%4) ..+3; the
        // transposed read hands lane i16 the 4 keys at column d0 + i16.
        const int key0 = 32 * kh + 16 * sp + 8 * g + 4 * hx;
        const int row = key0 + (i16 >> 2);
        const int col = d0 + 4 * (i16 & 3);
        const char* src = vbuf + ElemTraits<__bf16>::lds_off(row, col >> 3) + ((col & 7) << 1);
        s16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(src));
        bf16x4 tb = __builtin_bit_cast(bf16x4, t);
        for (int e = 0; e < 4; ++e) a[4 * hx + e] = tb[e];
      }
      acc.o[dh] = mfma_bf16(a, b, acc.o[dh]);
    }
  }
}
DEV void pv_half_f32(WaveAcc& acc, const char* vbuf, int kh, const f32x16& p, int lane) {
  const int g = lane >> 5;
  for (int t = 0; t < 16; ++t) {
    const float* vr = reinterpret_cast<const float*>(vbuf + (32 * kh + 2 * t + g) * ElemTraits<float>::ROWB);
    for (int dh = 0; dh < 2; ++dh) acc.o[dh] = mfma_f32(vr[32 * dh + (lane & 31)], p[t], acc.o[dh]);
  }
}

// Online-softmax update of one 64-key tile. s[kh] holds raw scores with
// masked entries at -inf; active[kh] says whether half kh was computed.
// Afterwards s[kh] holds the probabilities (relative to the new max).
template <class T>
DEV void softmax_tile(WaveAcc& acc, f32x16 (&s)[2], const bool (&active)[2], float c2) {
  float mx = -__builtin_inff();
  for (int kh = 0; kh < 2; ++kh)
    if (active[kh])
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[kh][j]);
  mx = fmaxf(mx, wave_xor32(mx));
  const float mnew = fmaxf(acc.m, mx);
  const float muse = mnew == -__builtin_inff() ? 0.f : mnew;
  const float alpha = __builtin_amdgcn_exp2f((acc.m - muse) * c2);
  const float moff = -muse * c2;
  float lsum = 0.f;
  for (int kh = 0; kh < 2; ++kh) {
    if (!active[kh]) continue;
    for (int j = 0; j < 16; ++j) {
      const float pj = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kh][j], c2, moff));
      s[kh][j] = pj;
      lsum += pj;
    }
  }
  acc.l = acc.l * alpha + lsum;
  if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
    for (int i = 0; i < 16; ++i) { acc.o[0][i] *= alpha; acc.o[1][i] *= alpha; }
  }
  acc.m = mnew;
}

// ----------------------------------------------------------------------------
// Cooperative tile loads: NT threads move 64 rows of K and V into LDS.

template <class T, int NT>
struct TileRegs {
  static constexpr int NC = KT * ElemTraits<T>::CPR / NT;  // chunks per thread per tensor
  uint4 k[NC];
  uint4 v[NC];
};

// Row of tile-local key `row`: returns the sequence position or -1 (padding).
struct BandRowMap {
  int kbase, kend, r, dil;
  DEV int pos(int row) const { int kk = kbase + row; return kk < kend ? r + kk * dil : -1; }
};
struct GlobalRowMap {
  const int* gidx;
  int base, ng;
  DEV int pos(int row) const { int i = base + row; return i < ng ? gidx[i] : -1; }
};
struct PlainRowMap {
  int kbase, kend;
  DEV int pos(int row) const { int kk = kbase + row; return kk < kend ? kk : -1; }
};

template <class T, int NT, class Map>
DEV void tile_fetch(TileRegs<T, NT>& tr, const char* kb, const char* vb, const Map& map, int tid) {
  constexpr int CPR = ElemTraits<T>::CPR;
  for (int u = 0; u < TileRegs<T, NT>::NC; ++u) {
    const int c = tid + NT * u;
    const int row = c / CPR, ch = c % CPR;
    const int pos = map.pos(row);
    if (pos >= 0) {
      const long off = (long)pos * ElemTraits<T>::ROWB + ch * 16;
      tr.k[u] = *reinterpret_cast<const uint4*>(kb + off);
      tr.v[u] = *reinterpret_cast<const uint4*>(vb + off);
    } else {
      tr.k[u] = make_uint4(0, 0, 0, 0);
      tr.v[u] = make_uint4(0, 0, 0, 0);
    }
  }
}

template <class T, int NT>
DEV void tile_commit(const TileRegs<T, NT>& tr, char* klds, char* vlds, int tid) {
  constexpr int CPR = ElemTraits<T>::CPR;
  for (int u = 0; u < TileRegs<T, NT>::NC; ++u) {
    const int c = tid + NT * u;
    const int row = c / CPR, ch = c % CPR;
    const int off = ElemTraits<T>::lds_off(row, ch);
    *reinterpret_cast<uint4*>(klds + off) = tr.k[u];
    *reinterpret_cast<uint4*>(vlds + off) = tr.v[u];
  }
}

template <class T>
DEV void pv_dispatch(WaveAcc& acc, const char* vbuf, int kh, const f32x16& p, int lane) {
  if constexpr (sizeof(T) == 2) pv_half(acc, vbuf, kh, p, lane);
  else pv_half_f32(acc, vbuf, kh, p, lane);
}

template <class T> DEV int key_of_reg(int j, int g) {
  if constexpr (sizeof(T) == 2) return key_of_reg16(j, g);
  else return key_of_reg32(j, g);
}

// Store the normalised O rows owned by this lane (query row `pos`).
DEV void store_o(__bf16* orow, const WaveAcc& acc, float inv, int g) {
  for (int dh = 0; dh < 2; ++dh)
    for (int a = 0; a < 4; ++a) {
      bf16x4 t;
      for (int e = 0; e < 4; ++e) t[e] = (__bf16)(acc.o[dh][4 * a + e] * inv);
      *reinterpret_cast<bf16x4*>(orow + 32 * dh + 8 * a + 4 * g) = t;
    }
}
DEV void store_o(float* orow, const WaveAcc& acc, float inv, int g) {
  for (int dh = 0; dh < 2; ++dh)
    for (int a = 0; a < 4; ++a) {
      f32x4 t;
      for (int e = 0; e < 4; ++e) t[e] = acc.o[dh][4 * a + e] * inv;
      *reinterpret_cast<f32x4*>(orow + 32 * dh + 8 * a + 4 * g) = t;
    }
}

// ----------------------------------------------------------------------------
// Band kernel (with the global columns folded in as extra key tiles).

template <class T>
__global__ __launch_bounds__(256) void band_fwd(BandParams p) {
  constexpr int ROWB = ElemTraits<T>::ROWB;
  constexpr int TILEB = KT * ROWB;
  __shared__ __attribute__((aligned(16))) char lds[2][2][TILEB];
  __shared__ int gmeta[2][2][KT];  // global tiles: key position, residue-local index

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, g = lane >> 5;
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int4 td = p.tiles[bid];
  const int bh = td.x, r = td.y, q0 = td.z;
  const HeadInfo hi = p.heads[bh % p.H];
  const int half = hi.half, right = hi.right, dil = hi.dil;
  const int nr = (p.n - r + dil - 1) / dil;
  const long base = (long)bh * p.n * ROWB;
  const char* kb = reinterpret_cast<const char*>(p.k) + base;
  const char* vb = reinterpret_cast<const char*>(p.v) + base;

  const int kbeg = max(0, q0 - half);
  const int kend = min(nr, q0 + BM + right);
  const int nband = (kend - kbeg + KT - 1) / KT;
  const int nglob = (p.ng + KT - 1) / KT;
  const int ntiles = nglob + nband;

  // this wave's query rows and key range (residue-local)
  const int qw0 = q0 + 32 * wave;
  const bool wave_live = qw0 < nr;
  const int qi = qw0 + (lane & 31);
  const bool row_ok = qi < nr;
  const int pos_q = r + min(qi, nr - 1) * dil;
  const int wk_lo = max(0, qw0 - half);
  const int wk_hi = min(nr - 1, qw0 + 31 + right);
  const int lim = p.causal ? pos_q : 0x7fffffff - 1;

  QFrag<T> qf;
  load_q(qf, reinterpret_cast<const T*>(reinterpret_cast<const char*>(p.q) + base + (long)pos_q * ROWB), g);
  WaveAcc acc;
  acc_init(acc);

  TileRegs<T, 256> tr;
  auto fetch = [&](int t) {
    if (t < nglob) {
      GlobalRowMap m{p.gidx, t * KT, p.ng};
      tile_fetch<T, 256>(tr, kb, vb, m, tid);
    } else {
      BandRowMap m{kbeg + (t - nglob) * KT, kend, r, dil};
      tile_fetch<T, 256>(tr, kb, vb, m, tid);
    }
  };
  auto commit = [&](int t, int buf) {
    tile_commit<T, 256>(tr, lds[buf][0], lds[buf][1], tid);
    if (t < nglob && tid < KT) {
      const int idx = t * KT + tid;
      int kp = 0x7fffffff, kr = NEG_SENTINEL;
      if (idx < p.ng) {
        kp = p.gidx[idx];
        const int dr = kp - r;
        if (dr >= 0 && dr % dil == 0) kr = dr / dil;
      }
      gmeta[buf][0][tid] = kp;
      gmeta[buf][1][tid] = kr;
    }
  };

  fetch(0);
  commit(0, 0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) fetch(t + 1);
    if (wave_live) {
      const char* kl = lds[buf][0];
      const char* vl = lds[buf][1];
      f32x16 s[2];
      bool active[2];
      const bool is_glob = t < nglob;
      const int tkey0 = is_glob ? t * KT : kbeg + (t - nglob) * KT;
      for (int kh = 0; kh < 2; ++kh) {
        const int k0 = tkey0 + 32 * kh;
        active[kh] = is_glob ? (k0 < p.ng) : (k0 <= wk_hi && k0 + 31 >= wk_lo);
        if (!active[kh]) continue;
        s[kh] = score_half(kl, kh, qf, lane);
        if (is_glob) {
          for (int j = 0; j < 16; ++j) {
            const int kk = 32 * kh + key_of_reg<T>(j, g);
            const int kp = gmeta[buf][0][kk], kr = gmeta[buf][1][kk];
            const bool inband = kr >= qi - half && kr <= qi + right;
            if (!(kp <= lim) || inband) s[kh][j] = -__builtin_inff();
          }
        } else {
          const bool interior = k0 >= qw0 + 31 - half && k0 + 31 <= qw0 + right && k0 + 31 < nr;
          if (!interior) {
            for (int j = 0; j < 16; ++j) {
              const int kk = k0 + key_of_reg<T>(j, g);
              if (kk < qi - half || kk > qi + right || kk >= nr) s[kh][j] = -__builtin_inff();
            }
          }
        }
      }
      if (active[0] || active[1]) {
        softmax_tile<T>(acc, s, active, p.c2);
        for (int kh = 0; kh < 2; ++kh)
          if (active[kh]) pv_dispatch<T>(acc, vl, kh, s[kh], lane);
      }
    }
    if (t + 1 < ntiles) commit(t + 1, buf ^ 1);
    __syncthreads();
  }

  if (wave_live) {
    const float ltot = acc.l + wave_xor32(acc.l);
    if (row_ok) {
      const float inv = 1.0f / ltot;
      T* orow = reinterpret_cast<T*>(reinterpret_cast<char*>(p.o) + base + (long)pos_q * ROWB);
      store_o(orow, acc, inv, g);
      if (p.lse && g == 0) p.lse[(long)bh * p.n + pos_q] = acc.m * p.scale + __logf(ltot);
    }
  }
}

// ----------------------------------------------------------------------------
// Global rows: partial attention of up to 32 global rows over one key chunk.
// One wave per workgroup; grid = nsplit * nqb * B*H, split index fastest.

template <class T>
__global__ __launch_bounds__(64) void global_rows_partial(GlobalParams p) {
  constexpr int ROWB = ElemTraits<T>::ROWB;
  constexpr int TILEB = KT * ROWB;
  __shared__ __attribute__((aligned(16))) char lds[2][TILEB];
  const int lane = threadIdx.x, g = lane >> 5;
  const int sp = blockIdx.x % p.nsplit;
  const int qb = (blockIdx.x / p.nsplit) % p.nqb;
  const int bh = blockIdx.x / (p.nsplit * p.nqb);
  const long base = (long)bh * p.n * ROWB;
  const char* kb = reinterpret_cast<const char*>(p.kg) + base;
  const char* vb = reinterpret_cast<const char*>(p.vg) + base;

  const int gi = qb * 32 + (lane & 31);
  const int gq = min(gi, p.ng - 1);
  const int pos_q = p.gidx[gq];
  // G is sorted: the last row of this block bounds the causal key range.
  const int gmax = p.gidx[min(qb * 32 + 31, p.ng - 1)];
  const int k_lo = sp * p.ksplit;
  int k_hi = min(p.n, k_lo + p.ksplit);
  if (p.causal) k_hi = min(k_hi, gmax + 1);
  const int lim = p.causal ? pos_q : 0x7fffffff - 1;

  QFrag<T> qf;
  load_q(qf, reinterpret_cast<const T*>(reinterpret_cast<const char*>(p.qg) + base + (long)pos_q * ROWB), g);
  WaveAcc acc;
  acc_init(acc);

  TileRegs<T, 64> tr;
  for (int k0 = k_lo; k0 < k_hi; k0 += KT) {
    PlainRowMap m{k0, k_hi};
    tile_fetch<T, 64>(tr, kb, vb, m, lane);
    __syncthreads();
    tile_commit<T, 64>(tr, lds[0], lds[1], lane);
    __syncthreads();
    f32x16 s[2];
    bool active[2];
    for (int kh = 0; kh < 2; ++kh) {
      const int kk0 = k0 + 32 * kh;
      active[kh] = kk0 < k_hi;
      if (!active[kh]) continue;
      s[kh] = score_half(lds[0], kh, qf, lane);
      const bool interior = kk0 + 31 < k_hi && (!p.causal || kk0 + 31 <= p.gidx[min(qb * 32, p.ng - 1)]);
      if (!interior) {
        for (int j = 0; j < 16; ++j) {
          const int kk = kk0 + key_of_reg<T>(j, g);
          if (kk >= k_hi || !(kk <= lim)) s[kh][j] = -__builtin_inff();
        }
      }
    }
    softmax_tile<T>(acc, s, active, p.c2);
    for (int kh = 0; kh < 2; ++kh)
      if (active[kh]) pv_dispatch<T>(acc, lds[1], kh, s[kh], lane);
  }

  const float ltot = acc.l + wave_xor32(acc.l);
  if (gi < p.ng) {
    const long slot = ((long)bh * p.ng + gi) * p.nsplit + sp;
    float* po = p.part_o + slot * HD;
    for (int dh = 0; dh < 2; ++dh)
      for (int a = 0; a < 4; ++a) {
        f32x4 t;
        for (int e = 0; e < 4; ++e) t[e] = acc.o[dh][4 * a + e];
        *reinterpret_cast<f32x4*>(po + 32 * dh + 8 * a + 4 * g) = t;
      }
    if (g == 0) {
      p.part_ml[slot * 2 + 0] = acc.m;
      p.part_ml[slot * 2 + 1] = ltot;
    }
  }
}

// Log-sum-exp merge of the key chunks of one global row; overwrites O and LSE.
// One wave per (global row, b*h), grid = ng * B*H; lane = d.
template <class T>
__global__ __launch_bounds__(64) void global_rows_merge(GlobalParams p) {
  const int gi = blockIdx.x % p.ng, bh = blockIdx.x / p.ng, d = threadIdx.x;
  const long slot0 = ((long)bh * p.ng + gi) * p.nsplit;
  float M = -__builtin_inff();
  for (int s = 0; s < p.nsplit; ++s) M = fmaxf(M, p.part_ml[(slot0 + s) * 2]);
  float L = 0.f, acc = 0.f;
  for (int s = 0; s < p.nsplit; ++s) {
    const float ms = p.part_ml[(slot0 + s) * 2];
    if (ms == -__builtin_inff()) continue;
    const float w = __builtin_amdgcn_exp2f((ms - M) * p.c2);
    L += w * p.part_ml[(slot0 + s) * 2 + 1];
    acc += w * p.part_o[(slot0 + s) * HD + d];
  }
  const int pos = p.gidx[gi];
  T* orow = reinterpret_cast<T*>(p.o) + ((long)bh * p.n + pos) * HD;
  orow[d] = (T)(acc / L);
  if (p.lse && d == 0) p.lse[(long)bh * p.n + pos] = M * p.scale + __logf(L);
}

}  // namespace swattn
