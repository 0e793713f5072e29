// Host side of the C ABI declared in include/swattn.h: validation, plan
// construction (residue-class tile schedule with per-head geometry, sorted
// global index list, global-row workspace) and the stream-ordered launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <limits>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "swattn.h"
#include "kernels.hpp"
#include "backward.hpp"
#include "backward_f32.hpp"
#include "project.hpp"

using namespace swattn;

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(SWATTN_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Global-row pass: keys are cut into chunks of ksplit (a multiple of 64,
// about four tiles) so that every (b*h, group of 128 global rows) yields a
// few independent blocks; at most MAX_SPLIT chunks.
void choose_split(int n, int* nsplit, int* ksplit) {
  int ks = 4 * KT;
  while ((n + ks - 1) / ks > MAX_SPLIT) ks += KT;
  *ksplit = ks;
  *nsplit = (n + ks - 1) / ks;
}

// Streamed global rows (one global token per item): about eight chunks per
// row, of 256 to 1024 keys (a multiple of the 128 keys a block takes per
// round); longer chunks only where 1024-key chunks would exceed MAX_SPLIT.
void choose_stream_split(int n, int* nsplit, int* ksplit) {
  int ks = ((n + 7) / 8 + 127) / 128 * 128;
  ks = std::max(256, std::min(1024, ks));
  while ((n + ks - 1) / ks > MAX_SPLIT) ks += 128;
  *ksplit = ks;
  *nsplit = (n + ks - 1) / ks;
}

}  // namespace

struct swattn_plan {
  int B, H, n, d, causal, ng, dtype, device;
  int nband_blocks;       // band workgroups (explicit tiles, or the uniform decode)
  int uni_half, uni_right, uni_dil, uni_nqb;  // every head alike: no tile list
  int nsplit, ksplit, nqb, ngroup, nglob_blocks;
  int gstream;            // global rows by global_row_stream (bf16, |G| <= 1 per item)
  int gfuse;              // gstream, folded in the kernel (no key split): no global_rows_merge
  int bwd_gstream;        // backward: global row and column streamed (bf16, |G| <= 1 per item)
  int* gcount;            // [B*H] arrival counters of the fused fold, zero between launches
  int parts;              // key split of the band tiles (1: none)
  float* band_part;       // [B*H*n][parts][68] partials, NULL without a split
  void* dev_mem;          // one allocation, carved below
  TileRec* tiles;         // [nband_blocks], NULL with the uniform decode
  int* gidx;              // [n_global]: one sorted set, or the items' sorted sets
  int* goff;              // [B+1] offsets of the items' sets, NULL with one set
  bool per_item;
  float* part_o;          // [B*H][ng][nsplit][64]
  float* part_ml;         // [B*H][ng][nsplit][2]
  float* bwd_lse2;        // [B*H][n] backward row statistics (bf16 plans)
  float* bwd_dd;          // [B*H][n]
  // backward, global tokens (bf16 plans with n_global > 0)
  int ngp, ng32, nchunk, gcol_qc, nkgb, n_gkv, n_gcol;
  int bwd_nsplit, bwd_ksplit, n_gq;  // dQg blocks: key chunks (no more than the forward's)
  float* bwd_glse2;       // [B*H][ngp], +inf padding
  float* bwd_gdd;         // [B*H][ngp], 0 padding
  float* bwd_part_gkv;    // [B*H][nchunk][ng32][128]
  HeadGeom* bwd_heads;    // [H]
  // measurement hooks
  static constexpr int kMaxTimed = 4096;
  std::vector<hipEvent_t> ev;  // [kMaxTimed][4]: band start/stop, global start/stop
  int ntimed = 0;
};

extern "C" const char* swattn_status_string(int status) {
  switch (status) {
    case SWATTN_OK: return "SWATTN_OK";
    case SWATTN_ERR_INVALID_ARG: return "SWATTN_ERR_INVALID_ARG";
    case SWATTN_ERR_UNSUPPORTED: return "SWATTN_ERR_UNSUPPORTED";
    case SWATTN_ERR_HIP: return "SWATTN_ERR_HIP";
    case SWATTN_ERR_ALIGNMENT: return "SWATTN_ERR_ALIGNMENT";
    default: return "SWATTN_UNKNOWN_STATUS";
  }
}

extern "C" const char* swattn_last_error(void) { return g_last_error.c_str(); }

namespace {

// Everything the forward needs that follows from the parameters alone
// (host side, no device memory): validated geometry, the sorted global
// sets, the band tile schedule, the key split and the global-row chunks.
struct Schedule {
  int ng_max = 0;
  bool per_item = false;
  std::vector<int> G, goff;
  std::vector<TileRec> tiles;  // empty when every head has the same geometry
  std::vector<int> half, dil;
  long nband_blocks = 0;
  int parts = 1;
  int cus = 256;
  int nsplit = 0, ksplit = 0, nqb = 0, ngroup = 0;
  int stream = 0;  // global rows by global_row_stream
  int fuse = 0;    // stream, folded inside the kernel
  long nglob_blocks = 0;
};

int make_schedule(const swattn_params* p, Schedule* sc) {
  if (!p) return fail(SWATTN_ERR_INVALID_ARG, "params must not be NULL");
  if (p->batch < 1 || p->heads < 1) return fail(SWATTN_ERR_INVALID_ARG, "batch and heads must be >= 1");
  if (p->n < 1 || p->n > (1 << 24)) return fail(SWATTN_ERR_INVALID_ARG, "n must be in [1, 2^24]");
  if (p->causal != 0 && p->causal != 1) return fail(SWATTN_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (p->key_split < 0 || p->key_split > MAX_KEY_SPLIT)
    return fail(SWATTN_ERR_INVALID_ARG, "key_split must be in [0, 16]");
  if (!p->window || !p->dilation) return fail(SWATTN_ERR_INVALID_ARG, "window and dilation must not be NULL");
  for (int h = 0; h < p->heads; ++h) {
    if (p->window[h] < 0 || (p->window[h] & 1))
      return fail(SWATTN_ERR_INVALID_ARG, "window[" + std::to_string(h) + "] must be even and >= 0");
    if (p->dilation[h] < 1)
      return fail(SWATTN_ERR_INVALID_ARG, "dilation[" + std::to_string(h) + "] must be >= 1");
  }
  const bool per_item = p->global_offsets != nullptr;
  const long gmax_total = per_item ? (long)p->batch * p->n : (long)p->n;
  if (p->n_global < 0 || p->n_global > gmax_total)
    return fail(SWATTN_ERR_INVALID_ARG, per_item ? "n_global must be in [0, batch*n]" : "n_global must be in [0, n]");
  if (p->n_global > 0 && !p->global_idx) return fail(SWATTN_ERR_INVALID_ARG, "global_idx must not be NULL when n_global > 0");
  // G: one sorted set, or the items' sorted sets one after another (goff)
  std::vector<int> G, goff;
  int ng_max = p->n_global;
  if (per_item) {
    goff.assign(p->global_offsets, p->global_offsets + p->batch + 1);
    if (goff[0] != 0 || goff[p->batch] != p->n_global)
      return fail(SWATTN_ERR_INVALID_ARG, "global_offsets must start at 0 and end at n_global");
    ng_max = 0;
    for (int b = 0; b < p->batch; ++b) {
      if (goff[b + 1] < goff[b]) return fail(SWATTN_ERR_INVALID_ARG, "global_offsets must not decrease");
      if (goff[b + 1] - goff[b] > p->n) return fail(SWATTN_ERR_INVALID_ARG, "an item's global set is larger than n");
      ng_max = std::max(ng_max, goff[b + 1] - goff[b]);
    }
  } else {
    goff = {0, p->n_global};
  }
  if (p->n_global > 0) G.assign(p->global_idx, p->global_idx + p->n_global);
  for (size_t b = 0; b + 1 < goff.size(); ++b) {
    auto s0 = G.begin() + goff[b], s1 = G.begin() + goff[b + 1];
    for (auto it = s0; it != s1; ++it)
      if (*it < 0 || *it >= p->n) return fail(SWATTN_ERR_INVALID_ARG, "global index out of [0, n)");
    std::sort(s0, s1);
    if (std::adjacent_find(s0, s1) != s1) return fail(SWATTN_ERR_INVALID_ARG, "global_idx repeats an index");
  }
  if (p->d != HD) return fail(SWATTN_ERR_UNSUPPORTED, "only d = 64 is supported");
  if (p->dtype != SWATTN_BF16 && p->dtype != SWATTN_FP32) return fail(SWATTN_ERR_UNSUPPORTED, "unknown dtype");
  const long bh = (long)p->batch * p->heads;
  if (bh * p->n > (1L << 31)) return fail(SWATTN_ERR_UNSUPPORTED, "batch*heads*n must be <= 2^31");
  // The merge grid has |G| * B*H <= B*H*n <= 2^31 blocks; the forward grid
  // is checked below.

  // per-head geometry; a window or dilation beyond n behaves as if clipped to n
  std::vector<int> half(p->heads), dil(p->heads);
  bool uniform = true;
  for (int h = 0; h < p->heads; ++h) {
    half[h] = std::min(p->window[h] / 2, p->n);
    dil[h] = std::min(p->dilation[h], p->n);
    uniform = uniform && half[h] == half[0] && dil[h] == dil[0];
  }
  // tile schedule: (b, h, residue r, 128-row block), neighbours adjacent.
  // With one geometry for all heads the kernel decodes the block index
  // itself (residue classes share one block count; a block past the end of
  // a shorter class does nothing).
  std::vector<TileRec> tiles;
  long nband_blocks = 0;
  if (uniform) {
    const long nqb = ((p->n + dil[0] - 1) / dil[0] + BM - 1) / BM;
    nband_blocks = bh * dil[0] * nqb;
  } else {
    for (int b = 0; b < p->batch; ++b)
      for (int h = 0; h < p->heads; ++h)
        for (int r = 0; r < dil[h]; ++r) {
          const int nr = (p->n - r + dil[h] - 1) / dil[h];
          for (int q0 = 0; q0 < nr; q0 += BM)
            tiles.push_back(TileRec{b * p->heads + h, r, q0, nr, half[h], p->causal ? 0 : half[h], dil[h], 0});
        }
    nband_blocks = (long)tiles.size();
  }
  // Key split: with fewer band workgroups than half the CUs the forward is
  // one short round of latency-bound workgroups; sharing each tile's keys
  // over two workgroups (merged afterwards) then pays (the LED decoder's
  // 96 tiles: 19.2 -> 17.2 us). Larger grids lose more to the partials'
  // traffic and the merge than they gain (one 4096-token sequence, 384
  // tiles: 19.8 -> 26.5 us), so they are not split unless asked.
  int cus = 256;
  {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      cus = 256;
  }
  int parts = p->key_split > 0 ? p->key_split : 1;
  if (p->key_split == 0 && nband_blocks > 0 && 2 * nband_blocks < cus) {
    double avg_tiles = 0;  // key tiles per band tile, on average
    if (uniform) {
      const int nr0 = (p->n + dil[0] - 1) / dil[0];
      avg_tiles = std::min<double>((nr0 + KT - 1) / KT,
                                   (double)(BM + half[0] + (p->causal ? 0 : half[0]) + KT - 1) / KT);
    } else {
      for (const TileRec& t : tiles) {
        const int kb = std::max(0, t.q0 - t.half), ke = std::min(t.nr, t.q0 + BM + t.right);
        avg_tiles += (double)((ke - kb + KT - 1) / KT);
      }
      avg_tiles /= (double)tiles.size();
    }
    if (avg_tiles >= 4) parts = 2;
  }
  const size_t split_bytes = parts > 1 ? (size_t)bh * p->n * parts * PART_STRIDE * sizeof(float) : 0;
  if (split_bytes > ((size_t)1 << 30)) return fail(SWATTN_ERR_UNSUPPORTED, "key split workspace above 1 GiB");
  if (nband_blocks * parts > 0x7fffffffL) return fail(SWATTN_ERR_UNSUPPORTED, "too many tiles");

  // the backward launch holds two blocks per band tile
  if (2 * nband_blocks > 0x7fffffffL) return fail(SWATTN_ERR_UNSUPPORTED, "too many tiles");
  sc->ng_max = ng_max;
  sc->per_item = per_item && ng_max > 0;
  sc->G = std::move(G);
  sc->goff = std::move(goff);
  sc->tiles = std::move(tiles);
  sc->half = std::move(half);
  sc->dil = std::move(dil);
  sc->nband_blocks = nband_blocks;
  sc->parts = parts;
  sc->cus = cus;
  sc->nqb = (ng_max + 31) / 32;
  sc->ngroup = (sc->nqb + BAND_WAVES - 1) / BAND_WAVES;
  if (ng_max > 0) {
    sc->stream = p->dtype == SWATTN_BF16 && ng_max == 1;
    // without a key split the band blocks leave the global row to the
    // streaming blocks, whose last one per (batch, head) folds the chunks
    sc->fuse = sc->stream && parts == 1;
    if (sc->stream) choose_stream_split(p->n, &sc->nsplit, &sc->ksplit);
    else choose_split(p->n, &sc->nsplit, &sc->ksplit);
    sc->nglob_blocks = (long)sc->nsplit * sc->ngroup * bh;
    if (sc->nglob_blocks + nband_blocks * parts > 0x7fffffffL) return fail(SWATTN_ERR_UNSUPPORTED, "too many blocks");
  }
  return SWATTN_OK;
}

}  // namespace

extern "C" int swattn_create(const swattn_params* p, swattn_plan** out) {
  g_last_error.clear();
  if (!p || !out) return fail(SWATTN_ERR_INVALID_ARG, "params and out must not be NULL");
  Schedule sc;
  if (const int rc = make_schedule(p, &sc)) return rc;
  const long bh = (long)p->batch * p->heads;
  const int ng_max = sc.ng_max;
  const long nband_blocks = sc.nband_blocks;
  const int parts = sc.parts;
  const std::vector<int>& G = sc.G;
  const std::vector<int>& goff = sc.goff;
  const std::vector<TileRec>& tiles = sc.tiles;
  const std::vector<int>& half = sc.half;
  const std::vector<int>& dil = sc.dil;
  const size_t split_bytes = parts > 1 ? (size_t)bh * p->n * parts * PART_STRIDE * sizeof(float) : 0;

  swattn_plan* pl = new (std::nothrow) swattn_plan();
  if (!pl) return fail(SWATTN_ERR_HIP, "host allocation failed");
  pl->B = p->batch; pl->H = p->heads; pl->n = p->n; pl->d = p->d;
  pl->causal = p->causal; pl->ng = ng_max; pl->dtype = p->dtype;
  pl->per_item = sc.per_item;
  pl->nband_blocks = (int)nband_blocks;
  pl->parts = parts;
  pl->band_part = nullptr;
  pl->uni_half = half[0];
  pl->uni_right = p->causal ? 0 : half[0];
  pl->uni_dil = dil[0];
  pl->uni_nqb = ((p->n + dil[0] - 1) / dil[0] + BM - 1) / BM;
  pl->nqb = sc.nqb;
  pl->ngroup = sc.ngroup;
  pl->nsplit = sc.nsplit;
  pl->ksplit = sc.ksplit;
  pl->nglob_blocks = (int)sc.nglob_blocks;
  pl->gstream = sc.stream;
  pl->gfuse = sc.fuse;
  hipError_t e = hipGetDevice(&pl->device);
  if (e != hipSuccess) { delete pl; return hip_fail(e, "hipGetDevice"); }

  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t sz_tiles = al(sizeof(TileRec) * std::max<size_t>(tiles.size(), 1));
  const size_t sz_g = al(sizeof(int) * std::max<size_t>(G.size(), 1));
  const size_t sz_goff = al(sizeof(int) * goff.size());
  const size_t nslot = (size_t)bh * pl->ng * pl->nsplit;
  const size_t sz_po = al(sizeof(float) * HD * nslot);
  const size_t sz_pml = al(sizeof(float) * 2 * nslot);
  const bool bwd = pl->dtype == SWATTN_BF16;
  // per-row backward statistics (both dtypes; the fp32 backward uses D only)
  const size_t sz_stat = al(sizeof(float) * (size_t)bh * p->n);
  const bool bwd_g = bwd && pl->ng > 0;
  pl->ngp = bwd_g ? (pl->ng + KT - 1) / KT * KT : 0;
  pl->ng32 = bwd_g ? (pl->ng + 31) / 32 * 32 : 0;
  const bool small_g = pl->ng <= 32;
  pl->gcol_qc = GCOL_QC;
  if (small_g) pl->gcol_qc = std::min(GCOL_QC_MAX, std::max(GCOL_QC, (p->n / 4 + GCOL_QC - 1) / GCOL_QC * GCOL_QC));
  pl->nchunk = bwd_g ? (p->n + pl->gcol_qc - 1) / pl->gcol_qc : 0;
  // the dQg partials live in the forward's global-row workspace: at most as
  // many key chunks as the forward has
  pl->bwd_ksplit = pl->ksplit;
  if (bwd_g && small_g) pl->bwd_ksplit = std::max(pl->ksplit, GQ_KEYS_SMALL_G);
  pl->bwd_nsplit = bwd_g ? (p->n + pl->bwd_ksplit - 1) / pl->bwd_ksplit : 0;
  pl->n_gq = bwd_g ? (int)((long)pl->bwd_nsplit * pl->ngroup * bh) : 0;
  pl->nkgb = bwd_g ? ((pl->ng + 31) / 32 + BAND_WAVES - 1) / BAND_WAVES : 0;
  {
    // one global token per item: the global rows and columns are streamed
    // (bwd_grow_stream writes dKg, dVg with the dQg partials)
    pl->bwd_gstream = bwd_g && pl->ng == 1;
    const long n_gkv = bwd_g && !pl->bwd_gstream ? bh * ((p->n + BM * GKV_GROUPS - 1) / (BM * GKV_GROUPS)) : 0;
    const long n_gcol = bwd_g ? bh * (long)pl->nchunk * pl->nkgb : 0;
    const long nbwd = 2 * nband_blocks + (long)pl->n_gq + n_gkv + n_gcol;
    if (nbwd > 0x7fffffffL) {
      delete pl;
      return fail(SWATTN_ERR_UNSUPPORTED, "too many blocks");
    }
    pl->n_gkv = (int)n_gkv;
    pl->n_gcol = (int)n_gcol;
  }
  const size_t sz_gstat = al(sizeof(float) * (size_t)bh * pl->ngp);
  const size_t sz_gkv = al(sizeof(float) * (size_t)bh * pl->nchunk * pl->ng32 * 2 * HD);
  const size_t sz_heads = al(sizeof(HeadGeom) * p->heads);
  const size_t sz_split = al(split_bytes);
  const size_t sz_cnt = al(sizeof(int) * (sc.fuse ? bh : 1));
  const size_t total = sz_tiles + sz_g + sz_goff + sz_po + sz_pml + 2 * sz_stat + 2 * sz_gstat + sz_gkv + sz_heads +
                       sz_split + sz_cnt;
  e = hipMalloc(&pl->dev_mem, total);
  if (e != hipSuccess) { delete pl; return hip_fail(e, "hipMalloc(plan)"); }
  char* m = static_cast<char*>(pl->dev_mem);
  pl->tiles = tiles.empty() ? nullptr : reinterpret_cast<TileRec*>(m); m += sz_tiles;
  pl->gidx = reinterpret_cast<int*>(m); m += sz_g;
  pl->goff = pl->per_item ? reinterpret_cast<int*>(m) : nullptr; m += sz_goff;
  pl->part_o = reinterpret_cast<float*>(m); m += sz_po;
  pl->part_ml = reinterpret_cast<float*>(m); m += sz_pml;
  pl->bwd_lse2 = sz_stat ? reinterpret_cast<float*>(m) : nullptr; m += sz_stat;
  pl->bwd_dd = sz_stat ? reinterpret_cast<float*>(m) : nullptr; m += sz_stat;
  pl->bwd_glse2 = reinterpret_cast<float*>(m); m += sz_gstat;
  pl->bwd_gdd = reinterpret_cast<float*>(m); m += sz_gstat;
  pl->bwd_part_gkv = reinterpret_cast<float*>(m); m += sz_gkv;
  pl->bwd_heads = reinterpret_cast<HeadGeom*>(m); m += sz_heads;
  pl->band_part = sz_split ? reinterpret_cast<float*>(m) : nullptr; m += sz_split;
  pl->gcount = reinterpret_cast<int*>(m);
  e = hipMemset(pl->gcount, 0, sz_cnt);
  if (e == hipSuccess && !tiles.empty()) e = hipMemcpy(pl->tiles, tiles.data(), sizeof(TileRec) * tiles.size(), hipMemcpyHostToDevice);
  if (e == hipSuccess && !G.empty()) e = hipMemcpy(pl->gidx, G.data(), sizeof(int) * G.size(), hipMemcpyHostToDevice);
  if (e == hipSuccess && pl->goff) e = hipMemcpy(pl->goff, goff.data(), sizeof(int) * goff.size(), hipMemcpyHostToDevice);
  if (e == hipSuccess && bwd_g) {
    // padding rows of the global-row statistics: P = 0 and D = 0 for ever
    const std::vector<float> inf((size_t)bh * pl->ngp, std::numeric_limits<float>::infinity());
    const std::vector<float> zero((size_t)bh * pl->ngp, 0.f);
    e = hipMemcpy(pl->bwd_glse2, inf.data(), sizeof(float) * inf.size(), hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy(pl->bwd_gdd, zero.data(), sizeof(float) * zero.size(), hipMemcpyHostToDevice);
  }
  if (e == hipSuccess) {
    std::vector<HeadGeom> hg(p->heads);
    for (int h = 0; h < p->heads; ++h) hg[h] = HeadGeom{half[h], p->causal ? 0 : half[h], dil[h], 0};
    e = hipMemcpy(pl->bwd_heads, hg.data(), sizeof(HeadGeom) * hg.size(), hipMemcpyHostToDevice);
  }
  if (e != hipSuccess) {
    (void)hipFree(pl->dev_mem);
    delete pl;
    return hip_fail(e, "hipMemcpy(plan)");
  }
  *out = pl;
  return SWATTN_OK;
}

namespace {
void destroy_events(swattn_plan* pl) {
  for (hipEvent_t x : pl->ev) (void)hipEventDestroy(x);
  pl->ev.clear();
  pl->ntimed = 0;
}
}  // namespace

extern "C" int swattn_set_timing(swattn_plan* pl, int enable) {
  g_last_error.clear();
  if (!pl) return fail(SWATTN_ERR_INVALID_ARG, "plan must not be NULL");
  destroy_events(pl);
  if (!enable) return SWATTN_OK;
  pl->ev.resize((size_t)swattn_plan::kMaxTimed * 4, nullptr);
  for (auto& x : pl->ev) {
    hipError_t e = hipEventCreate(&x);
    if (e != hipSuccess) { x = nullptr; destroy_events(pl); return hip_fail(e, "hipEventCreate"); }
  }
  return SWATTN_OK;
}

extern "C" int swattn_kernel_times(swattn_plan* pl, float* band_ms, float* global_ms, int* count) {
  g_last_error.clear();
  if (!pl || !band_ms || !global_ms || !count) return fail(SWATTN_ERR_INVALID_ARG, "NULL argument");
  double sb = 0, sg = 0;
  const int nt = std::min(pl->ntimed, swattn_plan::kMaxTimed);
  for (int i = 0; i < nt && !pl->ev.empty(); ++i) {
    float a = 0, b = 0;
    hipError_t e = hipEventSynchronize(pl->ev[4 * i + 1]);
    if (e == hipSuccess) e = hipEventElapsedTime(&a, pl->ev[4 * i + 0], pl->ev[4 * i + 1]);
    if (e == hipSuccess && (pl->parts > 1 || (pl->ng > 0 && !pl->gfuse))) {
      e = hipEventSynchronize(pl->ev[4 * i + 3]);
      if (e == hipSuccess) e = hipEventElapsedTime(&b, pl->ev[4 * i + 2], pl->ev[4 * i + 3]);
    }
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    sb += a; sg += b;
  }
  *count = nt;
  *band_ms = nt ? (float)(sb / nt) : 0.f;
  *global_ms = nt ? (float)(sg / nt) : 0.f;
  pl->ntimed = 0;
  return SWATTN_OK;
}

extern "C" int swattn_destroy(swattn_plan* plan) {
  g_last_error.clear();
  if (!plan) return SWATTN_OK;
  destroy_events(plan);
  hipError_t e = hipFree(plan->dev_mem);
  delete plan;
  if (e != hipSuccess) return hip_fail(e, "hipFree(plan)");
  return SWATTN_OK;
}

namespace {

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

template <class T>
int launch(swattn_plan* pl, const void* q, const void* k, const void* v, const void* qg,
           const void* kg, const void* vg, void* o, float* lse, hipStream_t st) {
  const float scale = 0.125f;  // 1/sqrt(64)
  BandParams bp{};
  bp.q = q; bp.k = k; bp.v = v; bp.o = o; bp.lse = lse;
  bp.tiles = pl->tiles; bp.gidx = pl->gidx; bp.goff = pl->goff; bp.ng = pl->ng;
  bp.uni_half = pl->uni_half; bp.uni_right = pl->uni_right; bp.uni_dil = pl->uni_dil;
  bp.uni_nqb = pl->uni_nqb;
  bp.parts = pl->parts; bp.part = pl->band_part;
  bp.fair = pl->ng == 0 ? 1 : 0;
  bp.H = pl->H; bp.n = pl->n; bp.causal = pl->causal;
  bp.c2 = scale * LOG2E; bp.scale = scale;
  GlobalParams gp{};
  gp.qg = qg; gp.kg = kg; gp.vg = vg; gp.o = o; gp.lse = lse; gp.gidx = pl->gidx;
  gp.part_o = pl->part_o; gp.part_ml = pl->part_ml;
  gp.goff = pl->goff; gp.H = pl->H;
  gp.ng = pl->ng; gp.n = pl->n; gp.causal = pl->causal;
  gp.nsplit = pl->nsplit; gp.ksplit = pl->ksplit; gp.nqb = pl->nqb; gp.ngroup = pl->ngroup;
  gp.stream = pl->gstream;
  gp.fuse = pl->gfuse;
  gp.gcount = pl->gcount;
  bp.gskip = pl->gfuse;
  gp.c2 = scale * LOG2E; gp.scale = scale;

  const bool timed = !pl->ev.empty() && pl->ntimed < swattn_plan::kMaxTimed;
  hipEvent_t* ev = timed ? &pl->ev[4 * (size_t)pl->ntimed] : nullptr;
  if (timed) pl->ntimed++;
  // With timing on, events recorded on the stream around the launches
  // bracket the forward kernel (ev[0], ev[1]) and the merges after it (the
  // key-split merge and the global-row merge: ev[2], ev[3]). Each interval
  // covers the kernel's dispatch and its completion, including the cache
  // write-back at its end, as a kernel trace's per-dispatch duration does;
  // events attached to the launch itself leave that write-back out (about
  // 10 % less on the encoder shape).
  const int nfwd = pl->nband_blocks * pl->parts;
  const dim3 grid(nfwd + pl->nglob_blocks), block(256);
  hipError_t e = hipSuccess;
  if (timed) e = hipEventRecord(ev[0], st);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  if constexpr (sizeof(T) == 2) {
    if (gp.stream) hipLaunchKernelGGL((attn_fwd<T, true>), grid, block, 0, st, bp, gp, nfwd);
    else hipLaunchKernelGGL((attn_fwd<T, false>), grid, block, 0, st, bp, gp, nfwd);
  } else {
    hipLaunchKernelGGL((attn_fwd<T, false>), grid, block, 0, st, bp, gp, nfwd);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "launch attn_fwd");
  if (timed) e = hipEventRecord(ev[1], st);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  const bool merges = pl->parts > 1 || (pl->ng > 0 && !pl->gfuse);
  if (timed && merges) e = hipEventRecord(ev[2], st);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  if (pl->parts > 1) {
    // every row of O and LSE from its key parts (the rows of G are
    // overwritten by the global-row merge after it)
    const long rows = (long)pl->B * pl->H * pl->n;
    const dim3 bgrid((unsigned)((rows + 15) / 16));
    hipLaunchKernelGGL(band_merge<T>, bgrid, block, 0, st, bp, rows);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "launch band_merge");
  }
  if (pl->ng > 0 && !pl->gfuse) {
    const int nrows = pl->ng * pl->B * pl->H;  // <= B*H*n <= 2^31
    const dim3 mgrid((unsigned)((nrows + 3) / 4));
    hipLaunchKernelGGL(global_rows_merge<T>, mgrid, block, 0, st, (const float*)gp.part_ml,
                       (const float*)gp.part_o, gp.ng, gp.nsplit, nrows, gp);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "launch global_rows_merge");
  }
  if (timed && merges) e = hipEventRecord(ev[3], st);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  return SWATTN_OK;
}

}  // namespace

namespace {
// The plan's memory lives on the device it was created on; kernels go to the
// current device.
int check_device(const swattn_plan* pl) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != pl->device) return fail(SWATTN_ERR_INVALID_ARG, "the current device is not the plan's device");
  return SWATTN_OK;
}
}  // namespace

namespace {
// The tensor arguments of a forward: NULL-ness, alignment, no overlap of an
// output with an input.
int check_forward_args(long B, long H, long n, int dtype, int ng, const void* q, const void* k,
                       const void* v, const void* qg, const void* kg, const void* vg, const void* o,
                       const float* lse) {
  if (!q || !k || !v || !o) return fail(SWATTN_ERR_INVALID_ARG, "q, k, v and o must not be NULL");
  const bool want_g = ng > 0;
  if ((qg != nullptr) != want_g || (kg != nullptr) != want_g || (vg != nullptr) != want_g)
    return fail(SWATTN_ERR_INVALID_ARG, "qg, kg, vg must be non-NULL exactly when n_global > 0");
  const void* all[] = {q, k, v, qg, kg, vg, o, lse};
  for (const void* x : all)
    if (x && !aligned16(x)) return fail(SWATTN_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
  const size_t es = dtype == SWATTN_BF16 ? 2 : 4;
  const size_t nbytes = (size_t)B * H * n * HD * es;
  const void* ins[] = {q, k, v, qg, kg, vg};
  for (const void* x : ins)
    if (overlaps(o, nbytes, x, nbytes)) return fail(SWATTN_ERR_INVALID_ARG, "o overlaps an input");
  if (lse) {
    const size_t lb = (size_t)B * H * n * sizeof(float);
    for (const void* x : ins)
      if (overlaps(lse, lb, x, nbytes)) return fail(SWATTN_ERR_INVALID_ARG, "lse overlaps an input");
    if (overlaps(lse, lb, o, nbytes)) return fail(SWATTN_ERR_INVALID_ARG, "lse overlaps o");
  }
  return SWATTN_OK;
}
}  // namespace

extern "C" int swattn_forward(swattn_plan* pl, const void* q, const void* k, const void* v,
                              const void* qg, const void* kg, const void* vg, void* o,
                              float* lse, void* stream) {
  g_last_error.clear();
  if (!pl) return fail(SWATTN_ERR_INVALID_ARG, "plan must not be NULL");
  if (const int rc = check_forward_args(pl->B, pl->H, pl->n, pl->dtype, pl->ng, q, k, v, qg, kg, vg, o, lse))
    return rc;
  if (const int rc = check_device(pl)) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (pl->dtype == SWATTN_BF16) return launch<__bf16>(pl, q, k, v, qg, kg, vg, o, lse, st);
  return launch<float>(pl, q, k, v, qg, kg, vg, o, lse, st);
}

// ----------------------------------------------------------------------------
// Allocation-free forward. The tables a plan would hold (tile list, global
// sets) and the partial results its kernels exchange (global-row chunks,
// key-split parts) live in one file-scope device array instead; its address
// on each device is looked up once, with that device current, and used for
// every launch there. Small host tables reach it through the arguments of a
// copy kernel, so nothing is allocated and nothing host-side must outlive
// the call.

namespace {

constexpr size_t SCRATCH_BYTES = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
unsigned char* g_scratch_ptr[MAX_DEVICES] = {};

int scratch_on_current_device(unsigned char** out, int* dev_out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= MAX_DEVICES) return fail(SWATTN_ERR_UNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = static_cast<unsigned char*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  *dev_out = dev;
  return SWATTN_OK;
}

constexpr int UPLOAD_CHUNK = 2048;
struct UploadArgs {
  unsigned char* dst;
  int nbytes;
  unsigned char data[UPLOAD_CHUNK];
};

__global__ __launch_bounds__(256) void upload_bytes(UploadArgs a) {
  for (int i = threadIdx.x; i < a.nbytes; i += blockDim.x) a.dst[i] = a.data[i];
}

}  // namespace

extern "C" int swattn_forward_noalloc(const swattn_params* p, const void* q, const void* k,
                                      const void* v, const void* qg, const void* kg, const void* vg,
                                      void* o, float* lse, void* stream) {
  g_last_error.clear();
  if (!p) return fail(SWATTN_ERR_INVALID_ARG, "params must not be NULL");
  Schedule sc;
  if (const int rc = make_schedule(p, &sc)) return rc;
  if (const int rc = check_forward_args(p->batch, p->heads, p->n, p->dtype, sc.ng_max, q, k, v, qg, kg, vg,
                                        o, lse))
    return rc;
  unsigned char* base = nullptr;
  int dev = -1;
  if (const int rc = scratch_on_current_device(&base, &dev)) return rc;

  // layout in the scratch array (256-byte aligned pieces)
  const long bh = (long)p->batch * p->heads;
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t o_tiles = 0;
  const size_t o_g = o_tiles + al(sizeof(TileRec) * sc.tiles.size());
  const size_t o_goff = o_g + al(sizeof(int) * sc.G.size());
  const size_t o_cnt = o_goff + al(sizeof(int) * sc.goff.size());  // uploaded as zeros on every call
  const size_t o_po = o_cnt + al(sizeof(int) * (sc.fuse ? bh : 1));
  const size_t nslot = (size_t)bh * sc.ng_max * sc.nsplit;
  const size_t o_pml = o_po + al(sizeof(float) * HD * nslot);
  const size_t o_part = o_pml + al(sizeof(float) * 2 * nslot);
  const size_t split_bytes = sc.parts > 1 ? (size_t)bh * p->n * sc.parts * PART_STRIDE * sizeof(float) : 0;
  const size_t total = o_part + al(split_bytes);
  if (total > SCRATCH_BYTES)
    return fail(SWATTN_ERR_UNSUPPORTED, "swattn_forward_noalloc: this problem needs " + std::to_string(total) +
                                            " bytes of scratch, above the " + std::to_string(SCRATCH_BYTES) +
                                            "-byte static array (use a plan)");

  hipStream_t st = static_cast<hipStream_t>(stream);
  // the host tables, laid out as in the scratch array, through copy kernels
  std::vector<unsigned char> host(o_po, 0);
  if (!sc.tiles.empty()) std::memcpy(host.data() + o_tiles, sc.tiles.data(), sizeof(TileRec) * sc.tiles.size());
  if (!sc.G.empty()) std::memcpy(host.data() + o_g, sc.G.data(), sizeof(int) * sc.G.size());
  std::memcpy(host.data() + o_goff, sc.goff.data(), sizeof(int) * sc.goff.size());
  for (size_t off = 0; off < host.size(); off += UPLOAD_CHUNK) {
    UploadArgs ua;
    ua.dst = base + off;
    ua.nbytes = (int)std::min<size_t>(UPLOAD_CHUNK, host.size() - off);
    std::memcpy(ua.data, host.data() + off, (size_t)ua.nbytes);
    hipLaunchKernelGGL(upload_bytes, dim3(1), dim3(256), 0, st, ua);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "launch upload_bytes");
  }

  // a plan on the stack whose device pointers all point into the scratch array
  swattn_plan pl = swattn_plan();
  pl.B = p->batch; pl.H = p->heads; pl.n = p->n; pl.d = p->d;
  pl.causal = p->causal; pl.ng = sc.ng_max; pl.dtype = p->dtype; pl.device = dev;
  pl.nband_blocks = (int)sc.nband_blocks;
  pl.uni_half = sc.half[0];
  pl.uni_right = p->causal ? 0 : sc.half[0];
  pl.uni_dil = sc.dil[0];
  pl.uni_nqb = ((p->n + sc.dil[0] - 1) / sc.dil[0] + BM - 1) / BM;
  pl.nsplit = sc.nsplit; pl.ksplit = sc.ksplit; pl.nqb = sc.nqb; pl.ngroup = sc.ngroup;
  pl.gstream = sc.stream;
  pl.gfuse = sc.fuse;
  pl.nglob_blocks = (int)sc.nglob_blocks;
  pl.parts = sc.parts;
  pl.per_item = sc.per_item;
  pl.tiles = sc.tiles.empty() ? nullptr : reinterpret_cast<TileRec*>(base + o_tiles);
  pl.gidx = reinterpret_cast<int*>(base + o_g);
  pl.goff = sc.per_item ? reinterpret_cast<int*>(base + o_goff) : nullptr;
  pl.part_o = reinterpret_cast<float*>(base + o_po);
  pl.part_ml = reinterpret_cast<float*>(base + o_pml);
  pl.band_part = sc.parts > 1 ? reinterpret_cast<float*>(base + o_part) : nullptr;
  pl.gcount = reinterpret_cast<int*>(base + o_cnt);
  if (p->dtype == SWATTN_BF16) return launch<__bf16>(&pl, q, k, v, qg, kg, vg, o, lse, st);
  return launch<float>(&pl, q, k, v, qg, kg, vg, o, lse, st);
}

extern "C" int swattn_backward(swattn_plan* pl, const void* q, const void* k, const void* v,
                               const void* qg, const void* kg, const void* vg, const void* o,
                               const float* lse, const void* dout, void* dq, void* dk, void* dv,
                               void* dqg, void* dkg, void* dvg, void* stream) {
  g_last_error.clear();
  if (!pl) return fail(SWATTN_ERR_INVALID_ARG, "plan must not be NULL");
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv)
    return fail(SWATTN_ERR_INVALID_ARG, "q, k, v, o, lse, dout, dq, dk and dv must not be NULL");
  if (const int rc = check_device(pl)) return rc;
  const bool want_g = pl->ng > 0;
  const void* gs[] = {qg, kg, vg, dqg, dkg, dvg};
  for (const void* x : gs)
    if ((x != nullptr) != want_g)
      return fail(SWATTN_ERR_INVALID_ARG, "qg, kg, vg, dqg, dkg, dvg must be non-NULL exactly when n_global > 0");
  const void* all[] = {q, k, v, qg, kg, vg, o, lse, dout, dq, dk, dv, dqg, dkg, dvg};
  for (const void* x : all)
    if (x && !aligned16(x)) return fail(SWATTN_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
  const size_t nbytes = (size_t)pl->B * pl->H * pl->n * HD * (pl->dtype == SWATTN_BF16 ? 2 : 4);
  const size_t lb = (size_t)pl->B * pl->H * pl->n * sizeof(float);
  const void* ins[] = {q, k, v, qg, kg, vg, o, dout};
  void* outs[] = {dq, dk, dv, dqg, dkg, dvg};
  for (int a = 0; a < 6; ++a) {
    if (!outs[a]) continue;
    for (const void* x : ins)
      if (overlaps(outs[a], nbytes, x, nbytes)) return fail(SWATTN_ERR_INVALID_ARG, "a gradient overlaps an input");
    if (overlaps(outs[a], nbytes, lse, lb)) return fail(SWATTN_ERR_INVALID_ARG, "a gradient overlaps lse");
    for (int b = 0; b < a; ++b)
      if (overlaps(outs[a], nbytes, outs[b], nbytes)) return fail(SWATTN_ERR_INVALID_ARG, "two gradients overlap");
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const float scale = 0.125f;
  BwdParams bp;
  bp.q = q; bp.k = k; bp.v = v; bp.qg = qg; bp.kg = kg; bp.vg = vg;
  bp.o = o; bp.dout = dout; bp.lse = lse;
  bp.dq = dq; bp.dk = dk; bp.dv = dv; bp.dqg = dqg; bp.dkg = dkg; bp.dvg = dvg;
  bp.lse2 = pl->bwd_lse2; bp.dd = pl->bwd_dd;
  bp.glse2 = pl->bwd_glse2; bp.gdd = pl->bwd_gdd;
  bp.part_dqg = pl->part_o;  // the forward's global-row workspace has this shape
  bp.part_gkv = pl->bwd_part_gkv;
  bp.tiles = pl->tiles; bp.heads = pl->bwd_heads;
  bp.uni_half = pl->uni_half; bp.uni_right = pl->uni_right; bp.uni_dil = pl->uni_dil;
  bp.uni_nqb = pl->uni_nqb;
  bp.gidx = pl->gidx; bp.goff = pl->goff; bp.ng = pl->ng; bp.ngp = pl->ngp; bp.ng32 = pl->ng32;
  bp.n = pl->n; bp.H = pl->H; bp.causal = pl->causal;
  bp.nsplit = pl->bwd_nsplit; bp.ksplit = pl->bwd_ksplit; bp.nqb = pl->nqb; bp.ngroup = pl->ngroup;
  bp.nchunk = pl->nchunk; bp.gcol_qc = pl->gcol_qc; bp.nkgb = pl->nkgb;
  bp.nq = pl->nband_blocks;
  bp.n_gq = pl->n_gq;
  bp.n_gkv = pl->n_gkv; bp.n_gcol = pl->n_gcol;
  bp.gstream = pl->bwd_gstream;
  bp.c2 = scale * LOG2E; bp.scale = scale;
  const long rows = (long)pl->B * pl->H * pl->n;
  if (pl->dtype == SWATTN_FP32) {
    // the fp32 path: D, then dq/dqg per row and dk/dv/dkg/dvg per key
    hipLaunchKernelGGL(bwd_f32_prep, dim3((unsigned)((rows * 16 + 255) / 256)), dim3(256), 0, st, bp, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "launch bwd_f32_prep");
    hipLaunchKernelGGL(bwd_f32_rows, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, bp, rows);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "launch bwd_f32_rows");
    hipLaunchKernelGGL(bwd_f32_keys, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, bp, rows);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "launch bwd_f32_keys");
    return SWATTN_OK;
  }
  hipLaunchKernelGGL(bwd_prep, dim3((unsigned)((rows * 4 + 255) / 256)), dim3(256), 0, st, bp, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "launch bwd_prep");
  const dim3 mgrid(2 * bp.nq + bp.n_gq + bp.n_gkv + bp.n_gcol);
  if (bp.gstream) hipLaunchKernelGGL(bwd_main<true>, mgrid, dim3(256), 0, st, bp);
  else hipLaunchKernelGGL(bwd_main<false>, mgrid, dim3(256), 0, st, bp);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "launch bwd_main");
  if (pl->ng > 0) {
    hipLaunchKernelGGL(bwd_gred, dim3(pl->ng * pl->B * pl->H), dim3(256), 0, st, bp);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "launch bwd_gred");
  }
  return SWATTN_OK;
}

extern "C" int swattn_project(const void* x, const void* w, const void* bias, void* out,
                              int batch, int n, int d_model, int heads, int nproj, int dtype,
                              void* stream) {
  g_last_error.clear();
  if (!x || !w || !out) return fail(SWATTN_ERR_INVALID_ARG, "x, w and out must not be NULL");
  if (batch < 1 || n < 1 || heads < 1 || nproj < 1 || d_model < 1)
    return fail(SWATTN_ERR_INVALID_ARG, "batch, n, heads, nproj and d_model must be >= 1");
  if (dtype != SWATTN_BF16 && dtype != SWATTN_FP32) return fail(SWATTN_ERR_UNSUPPORTED, "unknown dtype");
  if (d_model % PJ_TK) return fail(SWATTN_ERR_UNSUPPORTED, "d_model must be a multiple of 32");
  const long M = (long)batch * n, N = (long)nproj * heads * HD;
  const long es = dtype == SWATTN_BF16 ? 2 : 4;  // element size
  // 32-bit byte offsets into x and w
  if (M * d_model * es >= (1L << 31) || N * d_model * es >= (1L << 31))
    return fail(SWATTN_ERR_UNSUPPORTED, "x and w must each be smaller than 2 GiB");
  for (const void* ptr : {x, w, bias, (const void*)out})
    if (ptr && !aligned16(ptr)) return fail(SWATTN_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
  const size_t xb = (size_t)M * d_model * es, wb = (size_t)N * d_model * es, ob = (size_t)M * N * es;
  if (overlaps(out, ob, x, xb) || overlaps(out, ob, w, wb) || overlaps(out, ob, bias, (size_t)N * es))
    return fail(SWATTN_ERR_INVALID_ARG, "out overlaps an input");
  if (dtype == SWATTN_FP32) {
    const long ntm = (M + 63) / 64;
    if (ntm * (N / HD) > 0x7fffffffL) return fail(SWATTN_ERR_UNSUPPORTED, "too many blocks");
    ProjParamsF32 pf;
    pf.x = static_cast<const float*>(x);
    pf.w = static_cast<const float*>(w);
    pf.bias = static_cast<const float*>(bias);
    pf.out = static_cast<float*>(out);
    pf.M = (int)M; pf.N = (int)N; pf.D = d_model; pf.n = n; pf.B = batch; pf.H = heads;
    pf.nph = (int)(N / HD);
    hipLaunchKernelGGL(proj_f32, dim3((unsigned)(ntm * pf.nph)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), pf);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "launch proj_f32");
    return SWATTN_OK;
  }
  int cus = 256;
  {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      cus = 256;
  }
  const int tg = proj_choose_tg(M, N, cus);  // workgroup shape (PjCfg)
  // 256-token workgroups: eight waves over 256 output features (one per CU),
  // whose staged W and x tiles serve twice the MFMA work of four waves over
  // 128 features, when that still gives at least two rounds of workgroups
  // (the encoder's and LED's six projections: 78 -> 74 us, 155 -> 141 us);
  // otherwise, and for 128-token workgroups, four waves over 128 features
  const long ntm4 = (M + 255) / 256, ntn4 = (N + 255) / 256;
  const int wn = tg == 4 && ntm4 * ntn4 >= 2L * cus ? 4 : 2;  // waves along the output features
  const long tm_tokens = 64L * tg, tn_feats = 64L * wn;
  const long ntm = (M + tm_tokens - 1) / tm_tokens, ntn_all = (N + tn_feats - 1) / tn_feats;
  if (ntm * ntn_all > 0x7fffffffL) return fail(SWATTN_ERR_UNSUPPORTED, "too many blocks");
  // With eight-wave tiles (one workgroup per CU) and a last round at most a
  // third full, the feature tiles past the last whole round go to a second
  // launch of 128 x 128 tiles, four times as many workgroups for their work,
  // so that the last round is not a few CUs running whole tiles (the
  // encoder's six projections, a quarter-full third round: 72.6-72.9 ->
  // 69.5-69.9 us; LED's, a half-full fifth round, ran 2.8 us slower split).
  long ntn = ntn_all;
  const long nt = ntm * ntn_all;
  if (wn == 4 && nt > cus && nt % cus != 0 && 3 * (nt % cus) <= cus) {
    const long whole = nt / cus * cus / ntm;  // feature tiles filling whole rounds
    if (whole >= 1) ntn = whole;
  }
  ProjParams pp;
  pp.x = static_cast<const __bf16*>(x);
  pp.w = static_cast<const __bf16*>(w);
  pp.bias = static_cast<const __bf16*>(bias);
  pp.out = static_cast<__bf16*>(out);
  pp.M = (int)M; pp.N = (int)N; pp.D = d_model; pp.n = n; pp.B = batch; pp.H = heads;
  pp.tg = tg; pp.ntm = (int)ntm; pp.ntn = (int)ntn; pp.nblocks = (int)(ntm * ntn); pp.feat_base = 0;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (tg == 4 && wn == 4)
    hipLaunchKernelGGL((proj_gemm<4, 4>), dim3((unsigned)pp.nblocks), dim3(512), 0, st, pp);
  else if (tg == 4)
    hipLaunchKernelGGL(proj_gemm<4>, dim3((unsigned)pp.nblocks), dim3(256), 0, st, pp);
  else
    hipLaunchKernelGGL(proj_gemm<2>, dim3((unsigned)pp.nblocks), dim3(256), 0, st, pp);
  if (ntn < ntn_all) {
    hipError_t e0 = hipGetLastError();
    if (e0 != hipSuccess) return hip_fail(e0, "launch proj_gemm");
    const long f0 = ntn * tn_feats;
    const long ntm2 = (M + 127) / 128, ntn2 = (N - f0 + 127) / 128;
    if (ntm2 * ntn2 > 0x7fffffffL) return fail(SWATTN_ERR_UNSUPPORTED, "too many blocks");
    pp.tg = 2; pp.ntm = (int)ntm2; pp.ntn = (int)ntn2; pp.nblocks = (int)(ntm2 * ntn2);
    pp.feat_base = (int)f0;
    hipLaunchKernelGGL(proj_gemm<2>, dim3((unsigned)pp.nblocks), dim3(256), 0, st, pp);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "launch proj_gemm");
  return SWATTN_OK;
}
