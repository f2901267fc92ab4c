// GPU side of libsbm (gfx950 / CDNA4): reference decode, token grouping and
// the fused grouped decode + matrix-vector kernel.
//
// [QMoE] = "QMoE: Practical Sub-1-Bit Compression of Trillion-Parameter Models",
// section "The GPU Decoding Kernel" (fused decode-and-multiply, per-row
// offsets, ternary grid, skipping experts without tokens) and "The Fixed-to-
// Variable Dictionary Code" (Figure 4 entry layout).
// [M8.5] = "M8.5 - Extreme Weight Compression and Representations", 0x08A
// (reference decoder semantics).
//
// Fused kernel design (gfx950, wave64):
//  * Work: the output rows of every (expert, token chunk) item form one index
//    space; each persistent workgroup owns a contiguous, row-aligned slice, so
//    every output row is finished inside one workgroup (no global atomics).
//  * Stream fetch: a wave handles one block of SBM_BLOCK = 1024 codewords, 16
//    per lane, read as two range-checked 16-byte buffer loads per lane (2 KiB
//    per wave, coalesced), two blocks in flight per wave.  The block's start
//    position comes from the per-block offset table.
//  * Decode: the dictionary is held in LDS as one 60 KB table of 32-bit words
//    (the image built on the host); every entry has at most 3 nonzeros, so a
//    codeword yields its length and 3 "slots" (byte offsets of signed
//    activations, or of a zero) from one table read plus its sign bits.  Work
//    scales with nonzeros, never with the 28 symbols of a run.  Tables built
//    for other data hold entries with 4 nonzeros ([QMoE] "Limitations and
//    Trade-offs": a table per model); their 4-slot image (65.5 KB, 7-bit
//    slot fields) has kernel instances of its own.
//  * Positions: lane-local prefix of run lengths plus one wave scan (DPP).
//  * Accumulate: activations live in LDS as triples [-x, +x, 0] per column
//    (fp16, up to 4 rows interleaved), so each nonzero is one LDS read and one
//    fp32 add per row; zeros are never touched.  With cols >= 512 a lane (at
//    most 448 symbols) splits its sum at most once; row sums are formed from a
//    wave-wide prefix of lane sums.  Narrower rows take a per-codeword path.
//  * Epilogue: y = act(s_r * acc) per row and token (or, on the per-row
//    min/max grid, act(w_min * S1 + w_max * S2)), fp16 or fp32.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstddef>
#include <cstring>
#include <mutex>

#include "sbm_internal.h"

namespace sbm {

// ------------------------------------------------------------ constants
constexpr int kThreads = 1024;                // grouping kernel
constexpr int kWaves = kThreads / 64;
constexpr int kFThreads = 512;               // fused kernel: 8 waves, up to 256 VGPRs each
constexpr int kFWaves = kFThreads / 64;
constexpr int kK = 16;                // codewords per lane per block
static_assert(kK * 64 == SBM_BLOCK, "block = 64 lanes x kK codewords");
constexpr int kXPad = 48;             // columns past the row end: > 255/6, any slot byte stays inside
// Wide rows (cols >= kSmallCols): the first kXWrap columns are staged again
// after the row end, so a lane that runs into the next row (at most 448
// columns, plus any slot byte) reads that row's activations at the same base.
constexpr int kXWrap = 512;
constexpr int kSmallCols = 512;       // below this a lane (<= 448 symbols) may span several rows
// LDS: the decode tables are static arrays (compile-time addresses fold into
// instruction offsets); accumulators and activations are dynamic LDS.
struct __align__(16) LdsTables {
  uint32_t tab[kTabEntries];          // the image's decode table
};
static_assert(offsetof(DictImage, tab) % 16 == 0, "16B copies");
constexpr uint32_t kImageCopyU4 = kTabEntries / 4;
constexpr uint32_t kLdsFixed = (uint32_t)sizeof(LdsTables);
static_assert(kLdsFixed % 16 == 0, "align");
__shared__ LdsTables g_tab;
// The 4-slot table (dictionaries with 4-nonzero entries) is referenced only by
// the instances that read it, so the others do not reserve its LDS.
struct __align__(16) LdsTables4 {
  uint32_t tab[kTab4Entries];
};
static_assert(offsetof(DictImage4, tab) == offsetof(DictImage, tab), "one header layout");
static_assert(kTab4Entries % 4 == 0, "16B copies");
__shared__ LdsTables4 g_tab4;

// workspace layout (uint32 words)
constexpr uint32_t kWsHdr = 16;   // [0] error count, [1] n_items, [2] total item weight
constexpr int kMaxGrid = 1024;    // fused-kernel workgroups with precomputed slices
// Workgroups of a call: one per kRowsPerGroup output rows an upper bound of the
// items could hold, at most one per CU.
constexpr int64_t kRowsPerGroup = 16;
constexpr int kItemChangeBlocks = 20;   // measured: a chunk change costs ~16 one-token blocks
constexpr int kLayerItemChangeBlocks = 24;   // the same in a layer call's phases (best of 12..48 measured)
// Heavy experts (at least kMfmaMinTokens tokens) take the dense-tile MFMA path:
// items of up to kMfmaMaxTokens tokens, flagged in the item's token-count word.
constexpr uint32_t kItemMfma = 0x80000000u;
constexpr int kMfmaMinTokens = 16;
constexpr int kMfmaMaxTokens = 64;
constexpr uint32_t kMfmaWeight = 24;    // slice weight of one row of an MFMA item (measured, 1-token row = 4)
constexpr int kMaxRmax = 4096;    // rows per chunk
constexpr int kEpiRegs = (kMaxRmax + 2 + kFThreads - 1) / kFThreads;   // epilogue slots per thread
constexpr int kGroupInLds = 128;  // up to this many tokens are grouped inside the fused kernel
constexpr uint32_t kErrLayerWait = 0x10000000u, kErrDict = 0x20000000u, kErrBadDesc = 0x40000000u,
                   kErrBadImage = 0x80000000u;
constexpr uint32_t kErrCountMask = 0x0FFFFFFFu;   // bits 0-27: tokens with an expert id out of range
struct WsLayout {
  uint64_t cnt, start, chunk, perm, items, bounds, total_words;
};
__host__ __device__ inline WsLayout ws_layout(int64_t E, int64_t T) {
  WsLayout L;
  L.cnt = kWsHdr;
  L.start = L.cnt + E;
  L.chunk = L.start + E + 1;
  L.perm = L.chunk + E + 1;
  L.items = (L.perm + T + 3) & ~3ull;              // uint4 aligned
  L.bounds = L.items + 4 * (E + T);                // uint64[kMaxGrid + 1], 8-byte aligned
  L.total_words = L.bounds + 2 * (kMaxGrid + 1);
  return L;
}

struct FusedArgs {
  const uint16_t* codes;
  const uint32_t* row_off;
  const uint32_t* bstart;
  const uint16_t* scales;
  const sbm_matrix_desc* experts;
  const DictImage* image;
  const uint16_t* x;
  const int32_t* ids;
  void* y;
  uint32_t* ws;
  int32_t rows, cols, n_experts, n_tokens;
  int32_t group_in_lds; // 1: tokens grouped by every workgroup in LDS; 0: by group_kernel in ws
  int32_t grid;
  uint32_t item_cost;   // slice weight of an item change (row weights are 4..7)
  uint32_t flags;
  uint32_t colsB;       // 6 * cols
  uint32_t magic_s;
  uint64_t magic_m;     // exact division by colsB for numerators < 2^30
  int32_t rmax;         // rows per chunk (LDS accumulators)
  int32_t tcmax;        // interleaved activation rows per item (LDS capacity)
  int32_t titem;        // tokens per item: tcmax, or tcmax / 2 with the per-row min/max grid
  int32_t minmax;       // 1: per-row grid (w_min, w_max), each token staged as two rows
  int32_t xcols;        // staged columns per token (cols + pad)
  uint32_t lds_racc;    // byte offsets in LDS
  uint32_t lds_x;
  int32_t mfma_rows;    // rows per dense MFMA tile (16, 32 or 64); 0: heavy experts stay sparse
  int32_t det_shift;    // SBM_F_DETERMINISTIC: accumulator terms are rounded to multiples of 2^-det_shift
  uint32_t* err_out;    // if set, workgroup 0 copies the finished error word here
  // layer calls (several projections in one launch): lm bit 0, this phase's
  // output rows are written coherently at device scope and counted per token
  // in tok_done; bit 1, its input rows were written by the previous phase of
  // the same launch and are waited for (tok_wait reaching tok_expect) and
  // read coherently through a range-checked resource of x_bytes
  uint32_t lm;
  uint32_t* tok_done;
  const uint32_t* tok_wait;
  uint32_t tok_expect;
  uint32_t x_bytes;
  uint32_t* sync_err;   // the layer call's error accumulator (device-scope atomics only)
};

// Layer mode of the staging and epilogue code (template LM): 0 a single
// projection, no coherence; 3 a phase of a layer call, with the bits of a.lm
// deciding at run time whether its outputs are published (bit 0: stored
// coherently at device scope, per-token row counts raised after each chunk)
// and whether its inputs are waited for and read coherently (bit 1).
constexpr int kCpolSc1 = 16;                     // buffer-load cache policy: device-scope coherent
template <int LM>
__device__ __forceinline__ bool lm_out(const FusedArgs& a) {
  if constexpr (LM == 3) return (a.lm & 1u) != 0;
  else return false;
}
template <int LM>
__device__ __forceinline__ bool lm_in(const FusedArgs& a) {
  if constexpr (LM == 3) return (a.lm & 2u) != 0;
  else return false;
}

constexpr uint64_t kLayerWaitTicks = 2000000;    // 20 ms of the 100 MHz real-time counter

// Thread index through a volatile move: values derived from it are computed
// where they are used instead of being hoisted out of the phase loop.
__device__ __forceinline__ uint32_t tid_v() {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"((uint32_t)threadIdx.x));
  return r;
}
// ------------------------------------------------------------ wave helpers
// Inclusive scan over the 64 lanes of a wave (DPP row shifts, then the row
// broadcasts of lane 15 and lane 31).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false); // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false); // row_bcast:31
  return v;
}

__device__ __forceinline__ float wave_incl_scan_f(float f) {
  int v = __float_as_int(f);
  f += __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true));
  v = __float_as_int(f);
  f += __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true));
  v = __float_as_int(f);
  f += __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true));
  v = __float_as_int(f);
  f += __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true));
  v = __float_as_int(f);
  f += __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false));
  v = __float_as_int(f);
  f += __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false));
  return f;
}

__device__ __forceinline__ uint32_t div_magic_dev(uint32_t n, uint64_t m, uint32_t s) {
  return (uint32_t)(((uint64_t)n * m) >> s);
}

// ------------------------------------------------------------ decode_ref
// One thread per row: expand the row's codewords from the packed Figure-4
// words in order ([M8.5] 0x08A), writing symbols 0/1/2.
__global__ void decode_ref_kernel(const uint16_t* __restrict__ codes,
                                  const uint32_t* __restrict__ row_off, int32_t rows, int32_t cols,
                                  const uint32_t* __restrict__ words, uint8_t* __restrict__ out,
                                  uint32_t* __restrict__ bad_rows) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  const uint32_t b = row_off[r], e = row_off[r + 1];
  uint8_t* o = out + r * (int64_t)cols;
  int64_t pos = 0;
  bool ok = e >= b;
  for (uint32_t i = b; ok && i < e; ++i) {
    const uint32_t c = codes[i];
    const uint32_t w0 = words[2 * c], w1 = words[2 * c + 1];
    const uint32_t k = w0 & 0xFu;
    if (k == 0 || k > 14 || (w1 & 0xFu) != k) { ok = false; break; }
    for (uint32_t j = 0; j < 2 * k; ++j) {
      const uint32_t w = j < 14 ? w0 : w1;
      const uint32_t sh = 4 + 2 * (j < 14 ? j : j - 14);
      if (pos < cols) o[pos] = (uint8_t)((w >> sh) & 3u);
      ++pos;
    }
  }
  if (!ok || pos != cols) {
    if (bad_rows) atomicAdd(bad_rows, 1u);
  }
}

// ------------------------------------------------------------ grouping
// Single workgroup: histogram of expert ids, exclusive scans, scatter of token
// indices by expert, and the item list (expert, first token, token count) with
// at most tcmax tokens per item.  Experts without tokens get no item ([QMoE]:
// calls for experts that receive no tokens are skipped).
// Workgroup slices split the (item, row) space by estimated cost.  Item q,
// whose rows each weigh w_q, covers weighted positions [P_q, P_q + F + w_q *
// rows) with P_q = wpre_q * rows + q * F (wpre_q: exclusive prefix of w); the
// leading F charges the activation restaging and drain of an item change to
// the slice that contains it.  Positions map monotonically to global row
// indices (item * rows + row), so consecutive workgroups tile the row space.
// floor(n / d) for d > 0: a double quotient corrected to the exact floor when
// n < 2^52, else the 64-bit division.  On per-lane (vector) values this stays
// in VALU instructions.
__device__ __forceinline__ uint64_t udiv_small(uint64_t n, uint32_t d) {
  if (n < (1ull << 52)) {
    uint64_t q = (uint64_t)((double)n / (double)d);
    if (q * d > n) --q;
    else if ((q + 1) * d <= n) ++q;
    return q;
  }
  return n / d;
}

// A zero the compiler cannot see through: adding it makes a value per-lane,
// so arithmetic on it is done in vector registers instead of scalar ones
// (which would need vector -> scalar round trips for divisions).
__device__ __forceinline__ uint32_t vzero() {
  uint32_t z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return z;
}

// Slice arithmetic needs no exact quotient: a boundary is computed by the
// same expression in the two workgroups it separates, so any deterministic
// rounding that is monotone in n keeps the slices tiling the row space.  A
// double quotient stays in vector registers.
__device__ __forceinline__ uint64_t slice_div(uint64_t n, uint32_t d) {
  return (uint64_t)((double)n / (double)d);
}

__device__ __forceinline__ uint64_t boundary_in_item(uint64_t u, uint64_t pq, uint32_t q, uint32_t wq, uint32_t F,
                                                     uint64_t rows) {
  uint64_t r = 0;
  if (u > pq + F) {
    r = slice_div(u - pq - F + wq - 1, wq);
    if (r > rows) r = rows;
  }
  return (uint64_t)q * rows + r;
}

__device__ uint64_t weighted_boundary(const uint4* items, uint32_t n_items, uint32_t wtot, int32_t rows, uint32_t F,
                                      uint64_t u) {
  const uint64_t R = (uint64_t)rows;
  if (n_items == 0 || u >= (uint64_t)wtot * R + (uint64_t)n_items * F) return (uint64_t)n_items * R;
  uint32_t lo = 0, hi = n_items - 1;      // last item with P_q <= u
  while (lo < hi) {
    const uint32_t mid = (lo + hi + 1) / 2;
    if ((uint64_t)items[mid].w * R + (uint64_t)mid * F <= u) lo = mid;
    else hi = mid - 1;
  }
  const uint32_t w0 = items[lo].w;
  const uint32_t w1 = lo + 1 < n_items ? items[lo + 1].w : wtot;
  return boundary_in_item(u, (uint64_t)w0 * R + (uint64_t)lo * F, lo, w1 > w0 ? w1 - w0 : 1u, F, R);
}

// The dictionary tag of the decode image: the low 32 bits of its checksum.
__device__ __forceinline__ uint32_t image_tag(const FusedArgs& a) { return (uint32_t)a.image->checksum; }

// Why a matrix descriptor cannot be used for a call of this shape with this
// decode image: kErrBadDesc (shape, alignment), kErrDict (its codes were
// encoded with another dictionary, [M8.5] 0x08B), or 0.
__device__ __forceinline__ uint32_t desc_err(const sbm_matrix_desc& d, int32_t rows, int32_t cols, int32_t minmax,
                                             uint32_t dict_tag) {
  const bool shape = (d.code_base % SBM_CODE_ALIGN) == 0 && d.rows == rows && d.cols == cols &&
                     (!minmax || (d.scale_base & 1u) == 0);     // (w_min, w_max) pairs are read as one dword
  return (shape ? 0u : kErrBadDesc) | (d.dict_tag == dict_tag ? 0u : kErrDict);
}

constexpr uint32_t kRowWeight1 = 4;   // slice weight of a one-token row
// Relative cost of one output row of an item with nt tokens (processed with
// 1, 2 or 4 interleaved tokens); used to balance workgroup slices.
// (The min/max grid stages every token as two rows, so it weighs as twice the tokens.)
__host__ __device__ inline uint32_t item_weight(uint32_t nt, int32_t minmax) {
  if (nt & kItemMfma) return kMfmaWeight;
  const uint32_t n = minmax ? 2 * nt : nt;
  return n <= 1 ? kRowWeight1 : (n <= 2 ? 5u : 7u);   // measured: 4:5:7 beats 4:5:6, 4:5:8, 4:6:7, 4:6:8
}

__device__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh_tot, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(v);
  if (lane == 63) sh_tot[wave] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t run = 0;
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t t = sh_tot[w];
      sh_tot[w] = run;
      run += t;
    }
    sh_tot[kWaves] = run;
  }
  __syncthreads();
  const uint32_t out = sh_tot[wave] + inc - v;
  *total = sh_tot[kWaves];
  __syncthreads();
  return out;
}

__shared__ uint32_t sh_tot[kWaves + 1];
__device__ __forceinline__ void group_body(const int32_t* __restrict__ ids, int32_t T, int32_t E, int32_t titem,
                                           int32_t rows, int32_t cols, int32_t grid, uint32_t item_cost,
                                           int32_t mfma, int32_t minmax, const sbm_matrix_desc* __restrict__ experts,
                                           const DictImage* __restrict__ image, uint32_t* __restrict__ ws) {
  const WsLayout L = ws_layout(E, T);
  uint32_t* hdr = ws;
  uint32_t* cnt = ws + L.cnt;
  uint32_t* start = ws + L.start;
  uint32_t* chunk = ws + L.chunk;
  int32_t* perm = (int32_t*)(ws + L.perm);
  uint4* items = (uint4*)(ws + L.items);
  const uint32_t dict_tag = (uint32_t)image->checksum;
  for (int i = threadIdx.x; i < (int)kWsHdr; i += kThreads) hdr[i] = 0;
  for (int e = threadIdx.x; e < E; e += kThreads) cnt[e] = 0;
  __syncthreads();
  for (int t = threadIdx.x; t < T; t += kThreads) {
    const int32_t e = ids[t];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1u);
    else atomicAdd(&hdr[0], 1u);
  }
  __syncthreads();
  uint32_t carry_t = 0, carry_c = 0;
  for (int base = 0; base < E; base += kThreads) {
    const int e = base + threadIdx.x;
    const uint32_t c = e < E ? cnt[e] : 0u;
    const uint32_t span = (mfma && c >= (uint32_t)kMfmaMinTokens) ? (uint32_t)kMfmaMaxTokens : (uint32_t)titem;
    const uint32_t nch = (c + span - 1) / span;
    uint32_t tot_c, tot_n;
    const uint32_t ex_c = block_excl_scan(c, sh_tot, &tot_c);
    const uint32_t ex_n = block_excl_scan(nch, sh_tot, &tot_n);
    if (e < E) {
      start[e] = carry_t + ex_c;
      chunk[e] = carry_c + ex_n;
    }
    carry_t += tot_c;
    carry_c += tot_n;
  }
  if (threadIdx.x == 0) {
    start[E] = carry_t;
    chunk[E] = carry_c;
    hdr[1] = carry_c;
  }
  __syncthreads();
  // scatter: reuse cnt as the per-expert cursor
  for (int e = threadIdx.x; e < E; e += kThreads) cnt[e] = start[e];
  __syncthreads();
  for (int t = threadIdx.x; t < T; t += kThreads) {
    const int32_t e = ids[t];
    if (e >= 0 && e < E) perm[atomicAdd(&cnt[e], 1u)] = t;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kThreads) {
    const uint32_t s0 = start[e], n = start[e + 1] - s0;
    uint32_t q = chunk[e];
    const bool heavy = mfma && n >= (uint32_t)kMfmaMinTokens;
    const uint32_t span = heavy ? (uint32_t)kMfmaMaxTokens : (uint32_t)titem;
    for (uint32_t k = 0; k < n; k += span, ++q) {
      const uint32_t nt = ((n - k) < span ? (n - k) : span) | (heavy ? kItemMfma : 0u);
      items[q] = make_uint4((uint32_t)e, s0 + k, nt, item_weight(nt, minmax));
    }
    if (n) {
      const uint32_t err = desc_err(experts[e], rows, cols, minmax, dict_tag);
      if (err) atomicOr(&hdr[0], err);
    }
  }
  __syncthreads();
  // exclusive prefix of the per-row weights over items (.w), total in hdr[2]
  const uint32_t n_items = hdr[1];
  uint32_t carry = 0;
  for (uint32_t base = 0; base < n_items; base += kThreads) {
    const uint32_t q = base + threadIdx.x;
    const uint32_t wq = q < n_items ? items[q].w : 0u;
    uint32_t tot;
    const uint32_t ex = block_excl_scan(wq, sh_tot, &tot);
    if (q < n_items) items[q].w = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) hdr[2] = carry;
  __syncthreads();
  // contiguous weighted slices of the (item, row) space, one per fused workgroup
  uint64_t* bounds = (uint64_t*)(ws + L.bounds);
  const uint64_t wall = (uint64_t)carry * (uint64_t)rows + (uint64_t)n_items * item_cost;
  for (int g = threadIdx.x; g <= grid; g += kThreads)
    bounds[g] = weighted_boundary(items, n_items, carry, rows, item_cost, wall * (uint64_t)g / (uint64_t)grid);
}

__global__ __launch_bounds__(kThreads) void group_kernel(const int32_t* __restrict__ ids, int32_t T,
                                                         int32_t E, int32_t titem, int32_t rows, int32_t cols,
                                                         int32_t grid, uint32_t item_cost, int32_t mfma, int32_t minmax,
                                                         const sbm_matrix_desc* __restrict__ experts,
                                                         const DictImage* __restrict__ image,
                                                         uint32_t* __restrict__ ws) {
  group_body(ids, T, E, titem, rows, cols, grid, item_cost, mfma, minmax, experts, image, ws);
}

// ------------------------------------------------------------ fused kernel
// Copy of the decode image into LDS with direct-to-LDS loads issued at kernel
// entry: each wave moves 1 KB per instruction (lane l's 16 bytes land at the
// wave's LDS base + 16 l), so the copy holds no registers and completes while
// the tokens are grouped.  Wave 0 issues none of it: its loads (ids,
// descriptors, row offsets) form the prologue's dependent chain, and a wait
// for them would also wait for every load issued before them.  Readers wait
// for vmcnt(0) and then a barrier.
typedef __attribute__((address_space(3))) void lds_void_t;

template <int NS>
__device__ __forceinline__ void stage_tables_dma(const DictImage* __restrict__ im) {
  constexpr uint32_t kCopyU4 = NS == 3 ? kImageCopyU4 : kTab4Entries / 4;
  const uint4* src = (const uint4*)im->tab;
  uint4* dst = NS == 3 ? (uint4*)g_tab.tab : (uint4*)g_tab4.tab;
  const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave == 0) return;
  for (uint32_t q = wave - 1; q * 64 < kCopyU4; q += kFWaves - 1) {
    const uint32_t i = q * 64 + lane;
    if (i < kCopyU4)
      __builtin_amdgcn_global_load_lds((const void*)(src + i), (lds_void_t*)(dst + q * 64), 16, 0, 0);
  }
}

__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)

// acc += (float)x  with x the low / high fp16 half of v: one fp32 rounding.
__device__ __forceinline__ float acc_lo(float acc, uint32_t v) {
  float r;
  asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(v), "v"(acc));
  return r;
}
__device__ __forceinline__ float acc_hi(float acc, uint32_t v) {
  float r;
  asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(v), "v"(acc));
  return r;
}

// The x values of TC tokens at one slot byte address a (TC=1: fp16 in the low
// half; TC=2: one dword; TC=4: two dwords).
template <int TC>
struct XVal { uint32_t v[TC > 2 ? 2 : 1]; };

template <int TC>
__device__ __forceinline__ XVal<TC> lds_x(const unsigned char* smem, uint32_t a) {
  XVal<TC> r;
  if constexpr (TC == 1) r.v[0] = *(const uint16_t*)(smem + a);
  else if constexpr (TC == 2) r.v[0] = *(const uint32_t*)(smem + a);
  else {
    const uint2 t = *(const uint2*)(smem + a);
    r.v[0] = t.x;
    r.v[1] = t.y;
  }
  return r;
}

template <int TC>
__device__ __forceinline__ void acc_x(float* acc, const XVal<TC>& x) {
  if constexpr (TC == 1) acc[0] = acc_lo(acc[0], x.v[0]);
  else if constexpr (TC == 2) {
    acc[0] = acc_lo(acc[0], x.v[0]);
    acc[1] = acc_hi(acc[1], x.v[0]);
  } else {
    acc[0] = acc_lo(acc[0], x.v[0]);
    acc[1] = acc_hi(acc[1], x.v[0]);
    acc[2] = acc_lo(acc[2], x.v[1]);
    acc[3] = acc_hi(acc[3], x.v[1]);
  }
}

// The codewords of one block as this lane sees them, and the block's start
// position (bstart, in symbols from the matrix start).
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
constexpr int32_t kBufferFlags = 0x00020000;   // raw 32-bit buffer resource word 3 (gfx9 family)

struct BlockCodes {
  uint4 a, b;
  uint32_t bst;
};

// Everything a workgroup needs about one chunk: rows [ra, rb) of item q.
// The slice of workgroup b among n.  Workgroups are dealt to the 8 XCDs in
// turn (b mod 8), so this numbering gives each XCD a run of consecutive slices:
// the items of one expert, which all decode its codes, then mostly run on one
// XCD at about the same time and read the codes again from its L2.  A
// permutation of [0, n); workgroups b >= n (a launch holding more workgroups
// than this phase has slices) keep b, an empty slice.
__device__ __forceinline__ uint32_t xcd_slice(uint32_t b, uint32_t n) {
  if (b >= n) return b;
  const uint32_t x = b & 7u, per = n >> 3, extra = n & 7u;
  return x * per + (x < extra ? x : extra) + (b >> 3);
}

struct Chunk {
  uint32_t q, tb, nt;     // nt: token count (without the MFMA flag)
  int32_t ra, rb;
  uint32_t b0, b1;        // block range (inclusive); b0 > b1 when empty
  uint64_t code_base;
  uint32_t n_codes;
  uint64_t blk_base, scale_base, off_base;
  uint32_t seq0;          // first block sequence number of the chunk in its round
  bool ok;
  bool mfma;              // dense-tile MFMA item: no blocks in the round's sequence
};

// Rows [ra, rb) of item q.
__device__ __forceinline__ Chunk chunk_at(const FusedArgs& a, const uint4* items, uint32_t q, int32_t ra,
                                          int32_t rb) {
  Chunk ch;
  ch.q = q;
  ch.ra = ra;
  ch.rb = rb;
  const uint4 it = items[ch.q];
  ch.tb = it.y;
  ch.nt = it.z & ~kItemMfma;
  ch.mfma = (it.z & kItemMfma) != 0;
  const sbm_matrix_desc d = a.experts[it.x];
  ch.ok = desc_err(d, a.rows, a.cols, a.minmax, image_tag(a)) == 0;
  ch.code_base = d.code_base;
  ch.n_codes = d.n_codes;
  ch.blk_base = d.blk_base;
  ch.scale_base = d.scale_base;
  ch.off_base = d.off_base;
  ch.b0 = 1;
  ch.b1 = 0;
  if (ch.ok && !ch.mfma) {
    const uint32_t c0 = a.row_off[d.off_base + ch.ra], c1 = a.row_off[d.off_base + ch.rb];
    if (c1 > c0 && c1 <= d.n_codes) {
      ch.b0 = c0 / SBM_BLOCK;
      ch.b1 = (c1 - 1) / SBM_BLOCK;
    }
  }
  return ch;
}

// Codewords [b * SBM_BLOCK + 16 * lane, + 16) of a matrix's stream through a
// range-checked buffer resource: dwords wholly past the stream's end (rounded
// up to 4 bytes) read as zero, so every lane issues the same two loads and the
// compiler can count them (a per-lane tail path would make it wait for all
// loads in flight).  The rounding reads at most the rest of the dword that
// holds the last codeword; a codeword read past the end decodes to positions
// after the matrix's last row, which land in a clamped dummy accumulator.
__device__ __forceinline__ BlockCodes load_block(const FusedArgs& a, uint64_t code_base, uint32_t n_codes,
                                                 uint32_t b) {
  const uint32_t lane = threadIdx.x & 63;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.codes + code_base), (short)0, (int)((2u * n_codes + 3u) & ~3u),
                                        kBufferFlags);
  const uint32_t off = (b * SBM_BLOCK + lane * kK) * 2u;
  BlockCodes r;
  const i32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
  const i32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16u, 0, 0);
  r.a = make_uint4((uint32_t)lo.x, (uint32_t)lo.y, (uint32_t)lo.z, (uint32_t)lo.w);
  r.b = make_uint4((uint32_t)hi.x, (uint32_t)hi.y, (uint32_t)hi.z, (uint32_t)hi.w);
  return r;
}

// Decode-table index of codeword c for split H, given split7 = 7H: c itself
// below H, else H + (c - H) / 8, the codeword's group of 8 sign variants.
// (c + 7H) / 8 equals H + (c - H) / 8 from H on and is at least c below H,
// so one minimum covers both.
__device__ __forceinline__ uint32_t table_index(uint32_t c, uint32_t split7) {
  return min(c, (c + split7) >> 3);
}
// 2 * bit i of the sign index (c - H) & 7 = (c + 7H) & 7 into byte i (+2: the
// +x slot of the triple); with 4-slot words bit i into 7-bit field i.
template <int NS>
__device__ __forceinline__ uint32_t sign_spread(uint32_t c, uint32_t split7) {
  if constexpr (NS == 3) return (((c + split7) & 7u) * 0x8102u) & 0x20202u;
  else return (((c + split7) & 7u) * 0x1041u) & 0x4081u;
}
template <int NS>
__device__ __forceinline__ uint32_t table_word(uint32_t idx) {
  if constexpr (NS == 3) return g_tab.tab[idx];
  else return g_tab4.tab[idx];
}
// Byte offset of slot i within the codeword's first activation triple, and the
// run's length in bytes of triples (6 per column).
template <int NS>
__device__ __forceinline__ uint32_t slot_b(uint32_t s, int i) {
  if constexpr (NS == 3) return (s >> (8 * i)) & 0xFFu;
  else return ((s >> (7 * i)) & 0x7Fu) * 2u;
}
template <int NS>
__device__ __forceinline__ uint32_t run_b(uint32_t s) {
  if constexpr (NS == 3) return s >> 24;
  else return (s >> 28) * 12u;
}

// A block of SBM_BLOCK codewords, kK per lane, decoded: slot words with the
// signs added, the lane's total length and its start position (bytes).
struct DecBlock {
  uint32_t s[kK];
  uint32_t tot, pl;
};

// One table word per codeword, the signs of the 3-nonzero groups added back
// from the codeword's low bits; run lengths summed, lane start from a wave scan.
template <int NS>
__device__ __forceinline__ void decode_block(const BlockCodes& raw, uint32_t split7, DecBlock& d) {
  const uint32_t w[8] = {raw.a.x, raw.a.y, raw.a.z, raw.a.w, raw.b.x, raw.b.y, raw.b.z, raw.b.w};
  uint32_t c[kK];
#pragma unroll
  for (int j = 0; j < kK; ++j) c[j] = (j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xFFFFu);
#pragma unroll
  for (int j = 0; j < kK; ++j) d.s[j] = table_word<NS>(table_index(c[j], split7));
  uint32_t tot = 0;
#pragma unroll
  for (int j = 0; j < kK; ++j) {
    d.s[j] += sign_spread<NS>(c[j], split7);
    tot += run_b<NS>(d.s[j]);
  }
  d.tot = tot;
  d.pl = 6u * raw.bst + wave_incl_scan(tot) - tot;
}

// Row accumulators.  By default fp32 with LDS float atomics: the order in
// which waves add their partial sums varies from run to run, and so do the
// last bits of a row sum.  With SBM_F_DETERMINISTIC they are 64-bit integers
// in units of 2^-det_shift: each fp32 partial sum is rounded once to that
// grid and the integer sums are exact, so the result does not depend on the
// order of the additions.  The host picks det_shift so that no accumulator
// can overflow (every partial sum is below 2^28 for fp16 activations, and a
// row accumulator receives at most 3 per block touching the row).
__device__ __forceinline__ unsigned long long to_fixed(float v, int sh) {
  return (unsigned long long)(long long)rint(ldexp((double)v, sh));
}
__device__ __forceinline__ float from_fixed(unsigned long long q, int sh) {
  return (float)ldexp((double)(long long)q, -sh);
}
template <bool DET>
constexpr uint32_t acc_bytes() { return DET ? 8u : 4u; }
// Accumulator slot idx of activation row t.
template <bool DET>
__device__ __forceinline__ void racc_add(const FusedArgs& a, unsigned char* smem, int t, int32_t idx, float v) {
  unsigned char* base = smem + a.lds_racc + (uint32_t)t * (uint32_t)(a.rmax + 2) * acc_bytes<DET>();
  if constexpr (DET) atomicAdd((unsigned long long*)base + idx, to_fixed(v, a.det_shift));
  else atomicAdd((float*)base + idx, v);
}
// Read and clear.
template <bool DET>
__device__ __forceinline__ float racc_take(const FusedArgs& a, unsigned char* smem, int t, int32_t idx) {
  unsigned char* base = smem + a.lds_racc + (uint32_t)t * (uint32_t)(a.rmax + 2) * acc_bytes<DET>();
  if constexpr (DET) {
    unsigned long long* p = (unsigned long long*)base + idx;
    const unsigned long long q = *p;
    *p = 0ull;
    return from_fixed(q, a.det_shift);
  } else {
    float* p = (float*)base + idx;
    const float v = *p;
    *p = 0.f;
    return v;
  }
}
// Zero the accumulators of every activation row.
template <bool DET>
__device__ __forceinline__ void racc_clear(const FusedArgs& a, unsigned char* smem) {
  const uint32_t n4 = ((uint32_t)a.tcmax * (uint32_t)(a.rmax + 2) * acc_bytes<DET>() + 15u) / 16u;   // 16B-aligned
  uint4* r = (uint4*)(smem + a.lds_racc);
  for (uint32_t i = tid_v(); i < n4; i += kFThreads) r[i] = make_uint4(0, 0, 0, 0);
}

// Multiply-accumulate of one decoded block into the row accumulators.
template <int TC, bool SMALL, int NS, bool DET>
__device__ __forceinline__ void accumulate(const FusedArgs& a, const Chunk& ch, unsigned char* smem, const DecBlock& d) {
  const int lane = threadIdx.x & 63;
  const uint32_t tot = d.tot, pl = d.pl;
  uint32_t ls[kK];                   // codeword starts within the lane's span
  ls[0] = 0;
#pragma unroll
  for (int j = 1; j < kK; ++j) ls[j] = ls[j - 1] + run_b<NS>(d.s[j - 1]);
  const int32_t R = ch.rb - ch.ra;
  if constexpr (!SMALL) {
    const uint32_t rl = div_magic_dev(pl, a.magic_m, a.magic_s);
    const uint32_t colB = pl - rl * a.colsB;
    const uint32_t thr = a.colsB - colB;
    const uint32_t basex = colB + a.lds_x;    // row rl+1 continues into the wrap copy
    float acc[TC], snap[TC];
#pragma unroll
    for (int t = 0; t < TC; ++t) { acc[t] = 0.f; snap[t] = 0.f; }
    // Activation gathers in batches of kXB codewords: every address of a batch
    // is formed and its loads issued before the first sum, so up to 15 LDS
    // reads are in flight instead of three.
    constexpr int kXB = NS == 3 ? (TC == 4 ? 4 : 8) : 2;   // 4 slots: measured best at 2
#pragma unroll
    for (int j0 = 0; j0 < kK; j0 += kXB) {
      XVal<TC> xv[kXB][NS];
#pragma unroll
      for (int jj = 0; jj < kXB; ++jj) {
        const int j = j0 + jj;
        const uint32_t s = d.s[j];
        if constexpr (TC == 1) {
          // one add per slot: the byte operand is taken straight from s
          const uint32_t bx = basex + ls[j];
#pragma unroll
          for (int i = 0; i < NS; ++i) xv[jj][i] = lds_x<TC>(smem, bx + slot_b<NS>(s, i));
        } else {
          const uint32_t base = colB + ls[j];
#pragma unroll
          for (int i = 0; i < NS; ++i) xv[jj][i] = lds_x<TC>(smem, (base + slot_b<NS>(s, i)) * TC + a.lds_x);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int jj = 0; jj < kXB; ++jj) {
        const int j = j0 + jj;
#pragma unroll
        for (int i = 0; i < NS; ++i) acc_x<TC>(acc, xv[jj][i]);
        const bool first_row = ls[j] < thr;
#pragma unroll
        for (int t = 0; t < TC; ++t) snap[t] = first_row ? acc[t] : snap[t];
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // Row sums from a wave prefix of lane sums: a lane whose span reaches the
    // next row start closes row rl with E = prefix - (part past the boundary).
    const bool closes = tot >= thr;
    const int32_t i0 = (int32_t)rl - ch.ra + 1;
    const int32_t ia = i0 < 0 ? 0 : (i0 > R + 1 ? R + 1 : i0);
    const int32_t ib = (i0 + 1) < 0 ? 0 : ((i0 + 1) > R + 1 ? R + 1 : i0 + 1);
#pragma unroll
    for (int t = 0; t < TC; ++t) {
      const float S = wave_incl_scan_f(acc[t]);
      if (closes) {
        const float Ev = S - (acc[t] - snap[t]);
        racc_add<DET>(a, smem, t, ia, Ev);
        racc_add<DET>(a, smem, t, ib, -Ev);
      }
      if (lane == 63) racc_add<DET>(a, smem, t, closes ? ib : ia, S);
    }
  } else {
    // narrow rows: a lane may span several rows; locate every codeword's row
#pragma unroll
    for (int j = 0; j < kK; ++j) {
      const uint32_t p = pl + ls[j];
      const uint32_t r = div_magic_dev(p, a.magic_m, a.magic_s);
      const uint32_t base = p - r * a.colsB;
      const uint32_t s = d.s[j];
      uint32_t ad[NS];
#pragma unroll
      for (int i = 0; i < NS; ++i) ad[i] = (base + slot_b<NS>(s, i)) * TC + a.lds_x;
      float v[TC];
#pragma unroll
      for (int t = 0; t < TC; ++t) v[t] = 0.f;
#pragma unroll
      for (int i = 0; i < NS; ++i) acc_x<TC>(v, lds_x<TC>(smem, ad[i]));
      const int32_t i0 = (int32_t)r - ch.ra + 1;
      const int32_t ii = i0 < 0 ? 0 : (i0 > R + 1 ? R + 1 : i0);
#pragma unroll
      for (int t = 0; t < TC; ++t) racc_add<DET>(a, smem, t, ii, v[t]);
    }
  }
}

// Stage the activations of an item's tokens as triples [-x, +x, 0] per column,
// tokens interleaved: element (col, k, t) at byte ((3*col + k) * TC + t) * 2.
// Columns past cols are zero.  Each thread takes groups of 8 columns of all TC
// tokens (one 16-byte load per token) and writes 48*TC contiguous bytes.
// With the per-row min/max grid, rows 2u and 2u+1 both hold token u: row 2u as
// [-x, +x, 0] (its sum is A = S2 - S1 over the row's codes 1 and 2), row 2u+1
// as [+x, +x, 0] (B = S2 + S1), read at the same slot offsets.
template <int TC>
__device__ __forceinline__ void store_x_group(const FusedArgs& a, unsigned char* smem, int32_t c0,
                                              const uint32_t (&p)[TC][4]) {
  uint32_t o[12 * TC];
  if constexpr (TC == 1) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {           // columns 2m, 2m+1
      const uint32_t x = p[0][m];
      const uint32_t xl = x & 0xFFFFu, xh = x >> 16;
      o[3 * m + 0] = (xl ^ 0x8000u) | (xl << 16);          // [-x0, +x0]
      o[3 * m + 1] = (xh ^ 0x8000u) << 16;                 // [0, -x1]
      o[3 * m + 2] = xh;                                   // [+x1, 0]
    }
  } else {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
#pragma unroll
      for (int tp = 0; tp < TC / 2; ++tp) {                // token pair (2tp, 2tp+1)
        const uint32_t a0 = p[2 * tp][c / 2], a1 = p[2 * tp + 1][c / 2];
        const uint32_t pair = (c & 1) ? ((a0 >> 16) | (a1 & 0xFFFF0000u)) : ((a0 & 0xFFFFu) | (a1 << 16));
        o[(3 * c + 0) * (TC / 2) + tp] = pair ^ (a.minmax ? 0x00008000u : 0x80008000u);
        o[(3 * c + 1) * (TC / 2) + tp] = pair;
        o[(3 * c + 2) * (TC / 2) + tp] = 0u;
      }
    }
  }
  uint4* d = (uint4*)(smem + a.lds_x + (uint32_t)(6 * c0 * TC));
#pragma unroll
  for (int q = 0; q < 3 * TC; ++q) d[q] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
}

// Token place (within the item) of staged activation row t.
__device__ __forceinline__ uint32_t x_row_token(const FusedArgs& a, int t) {
  return a.minmax ? (uint32_t)t >> 1 : (uint32_t)t;
}

__device__ __forceinline__ bool x_vec(const FusedArgs& a) {
  return (a.cols % 8) == 0 && ((uintptr_t)a.x & 15u) == 0;
}

// Wide rows stage a wrap copy of their first columns after the row end.
__device__ __forceinline__ bool x_wrap(const FusedArgs& a) { return a.cols >= kSmallCols; }

// Source column of staged column c: c itself, or c - cols in the wrap copy
// (>= cols when there is none, i.e. zero).
__device__ __forceinline__ int32_t x_src(const FusedArgs& a, int32_t c, bool wrap) {
  return (wrap && c >= a.cols) ? c - a.cols : c;
}

// Activation loads: plain, or (inputs written by other workgroups of the
// same launch) device-scope coherent through a range-checked resource.
template <int LM>
__device__ __forceinline__ uint4 ld_x16(const FusedArgs& a, int64_t idx) {
  if (lm_in<LM>(a)) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)a.x, (short)0, (int)a.x_bytes, kBufferFlags);
    const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)idx * 2u, 0, kCpolSc1);
    return make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
  } else {
    return *(const uint4*)(a.x + idx);
  }
}
template <int LM>
__device__ __forceinline__ uint32_t ld_x2(const FusedArgs& a, int64_t idx) {
  if (lm_in<LM>(a)) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)a.x, (short)0, (int)a.x_bytes, kBufferFlags);
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (uint32_t)idx * 2u, 0, kCpolSc1);
  } else {
    return a.x[idx];
  }
}

// Inputs from the previous phase: wait until it has written all input rows of
// tokens perm[tb .. tb+nt) (each wave polls the nt counters; bounded by the
// real-time counter: on expiry the layer error bit is raised and the wave
// goes on, so the kernel always ends).  Other modes return at once.
template <int LM>
__device__ __forceinline__ void wait_tokens(const FusedArgs& a, const int32_t* perm, uint32_t tb, uint32_t nt) {
  if (lm_in<LM>(a)) {
    const uint32_t lane = tid_v() & 63;
    const bool mine = lane < nt;
    const uint32_t* p = a.tok_wait + (mine ? (uint32_t)perm[tb + lane] : 0u);
    const uint64_t t0 = wall_clock64();
    while (true) {
      const uint32_t v = mine ? __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : a.tok_expect;
      if (__all(v >= a.tok_expect)) break;
      if (wall_clock64() - t0 > kLayerWaitTicks) {
        if (lane == 0) __hip_atomic_fetch_or(a.sync_err, kErrLayerWait, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
}

// SBM_F_IN_BF16: two bf16 activations in a dword as the same two values in
// fp16 (exact for magnitudes in fp16's normal range, 2^-14 .. 65504; smaller
// ones round to fp16 subnormals).  The staged triples stay fp16, so the
// gathers and v_fma_mix accumulation are those of fp16 activations.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  const _Float16 lo = (_Float16)__uint_as_float(w << 16), hi = (_Float16)__uint_as_float(w & 0xFFFF0000u);
  return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

// fp16 pairs of staged columns c0 .. c0+7 of TC token rows (zero past the
// staged content or for tok < 0); bf16 activations are converted here.
template <int TC, int LM = 0>
__device__ __forceinline__ void load_x_group(const FusedArgs& a, const int32_t (&tok)[TC], int32_t c0, bool vec,
                                             bool wrap, uint32_t (&p)[TC][4]) {
  const int32_t s0 = x_src(a, c0, wrap);
#pragma unroll
  for (int t = 0; t < TC; ++t) {
    if (tok[t] >= 0 && s0 + 8 <= a.cols && vec) {
      const uint4 v = ld_x16<LM>(a, (int64_t)tok[t] * a.cols + s0);
      p[t][0] = v.x; p[t][1] = v.y; p[t][2] = v.z; p[t][3] = v.w;
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int32_t sl = x_src(a, c0 + 2 * m, wrap), sh = x_src(a, c0 + 2 * m + 1, wrap);
        uint32_t lo = 0, hi = 0;
        if (tok[t] >= 0 && sl < a.cols) lo = ld_x2<LM>(a, (int64_t)tok[t] * a.cols + sl);
        if (tok[t] >= 0 && sh < a.cols) hi = ld_x2<LM>(a, (int64_t)tok[t] * a.cols + sh);
        p[t][m] = lo | (hi << 16);
      }
    }
  }
  if (a.flags & SBM_F_IN_BF16) {
#pragma unroll
    for (int t = 0; t < TC; ++t)
#pragma unroll
      for (int m = 0; m < 4; ++m) p[t][m] = bf16x2_to_f16x2(p[t][m]);
  }
}

// SBM_F_IN_RMS: per-token sums of squares -> 1 / rms over the workgroup
// (wave scans, then the 8 wave totals in a fixed order; a zero row keeps scale 1).
__shared__ float s_ssq[kFWaves][4];

__device__ __forceinline__ float h2_ssq(uint32_t w) {
  const float lo = (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
  const float hi = (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  return lo * lo + hi * hi;
}

__device__ __forceinline__ uint32_t h2_scale(uint32_t w, float s) {
  const _Float16 lo = (_Float16)((float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu)) * s);
  const _Float16 hi = (_Float16)((float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)) * s);
  return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

template <int TC>
__device__ __forceinline__ void wg_inv_rms(const FusedArgs& a, const float (&ss)[TC], float (&inv)[TC]) {
  const int lane = tid_v() & 63, wave = tid_v() >> 6;
#pragma unroll
  for (int t = 0; t < TC; ++t) {
    const float S = wave_incl_scan_f(ss[t]);
    if (lane == 63) s_ssq[wave][t] = S;
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < TC; ++t) {
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kFWaves; ++w) tot += s_ssq[w][t];
    const float ms = tot / (float)a.cols;
    inv[t] = ms > 0.f ? 1.0f / sqrtf(ms) : 1.0f;
  }
  __syncthreads();
}

// Activations of the next item, requested before the drain barrier of the
// current chunk and stored after it: up to 4 groups of 8 columns x tokens
// per thread (4/TC groups of TC tokens), vector loads only.
struct XPre {
  uint4 v[4];
};

__device__ __forceinline__ bool x_prefetchable(const FusedArgs& a, int tc) {
  return x_vec(a) && a.xcols / 8 <= kFThreads * (4 / tc);
}

template <int TC, int LM = 0>
__device__ __forceinline__ void xpre_load(const FusedArgs& a, const int32_t* perm, uint32_t tb, uint32_t nt,
                                          XPre& r) {
  const int32_t n8 = a.xcols / 8;
#pragma unroll
  for (int j = 0; j < 4 / TC; ++j) {
    const int32_t c0 = 8 * ((int32_t)tid_v() + j * kFThreads);
    const int32_t s0 = x_src(a, c0, x_wrap(a));
#pragma unroll
    for (int t = 0; t < TC; ++t) {
      const uint32_t u = x_row_token(a, t);
      const int32_t tok = u < nt ? perm[tb + u] : -1;
      r.v[j * TC + t] = (tok >= 0 && s0 + 8 <= a.cols && c0 < 8 * n8)
                            ? ld_x16<LM>(a, (int64_t)tok * a.cols + s0) : make_uint4(0, 0, 0, 0);
    }
  }
}

template <int TC>
__device__ __forceinline__ void xpre_store(const FusedArgs& a, unsigned char* smem, XPre& r) {
  const int32_t n8 = a.xcols / 8;
  if (a.flags & SBM_F_IN_BF16) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      r.v[j] = make_uint4(bf16x2_to_f16x2(r.v[j].x), bf16x2_to_f16x2(r.v[j].y), bf16x2_to_f16x2(r.v[j].z),
                          bf16x2_to_f16x2(r.v[j].w));
  }
  float inv[TC];
  const bool rms = (a.flags & SBM_F_IN_RMS) != 0;
  if (rms) {
    float ss[TC];
#pragma unroll
    for (int t = 0; t < TC; ++t) ss[t] = 0.f;
#pragma unroll
    for (int j = 0; j < 4 / TC; ++j) {
      if (8 * ((int32_t)tid_v() + j * kFThreads) < a.cols) {     // the row itself, not its wrap copy
#pragma unroll
        for (int t = 0; t < TC; ++t) {
          const uint4 v = r.v[j * TC + t];
          ss[t] += h2_ssq(v.x) + h2_ssq(v.y) + h2_ssq(v.z) + h2_ssq(v.w);
        }
      }
    }
    wg_inv_rms<TC>(a, ss, inv);
  }
#pragma unroll
  for (int j = 0; j < 4 / TC; ++j) {
    const int32_t i = (int32_t)tid_v() + j * kFThreads;
    if (i < n8) {
      uint32_t p[TC][4];
#pragma unroll
      for (int t = 0; t < TC; ++t) {
        const uint4 v = r.v[j * TC + t];
        p[t][0] = v.x; p[t][1] = v.y; p[t][2] = v.z; p[t][3] = v.w;
        if (rms) {
#pragma unroll
          for (int m = 0; m < 4; ++m) p[t][m] = h2_scale(p[t][m], inv[t]);
        }
      }
      store_x_group<TC>(a, smem, 8 * i, p);
    }
  }
}

template <int TC, int LM = 0>
__device__ __forceinline__ void stage_x(const FusedArgs& a, unsigned char* smem, const int32_t* perm, uint32_t tb,
                        uint32_t nt) {
  wait_tokens<LM>(a, perm, tb, nt);
  if (x_prefetchable(a, TC)) {
    // one round trip: the rows stay in registers for the RMS scale
    XPre r;
    xpre_load<TC, LM>(a, perm, tb, nt, r);
    xpre_store<TC>(a, smem, r);
    return;
  }
  int32_t tok[TC];
#pragma unroll
  for (int t = 0; t < TC; ++t) tok[t] = x_row_token(a, t) < nt ? perm[tb + x_row_token(a, t)] : -1;
  const int32_t n8 = a.xcols / 8;
  const bool vec = x_vec(a);
  const bool rms = (a.flags & SBM_F_IN_RMS) != 0;
  float inv[TC];
  if (rms) {
    float ss[TC];
#pragma unroll
    for (int t = 0; t < TC; ++t) ss[t] = 0.f;
    for (int32_t i = tid_v(); 8 * i < a.cols; i += kFThreads) {     // the row itself, not its wrap copy
      uint32_t p[TC][4];
      load_x_group<TC, LM>(a, tok, 8 * i, vec, false, p);
#pragma unroll
      for (int t = 0; t < TC; ++t)
#pragma unroll
        for (int m = 0; m < 4; ++m) ss[t] += h2_ssq(p[t][m]);
    }
    wg_inv_rms<TC>(a, ss, inv);
  }
  for (int32_t i = tid_v(); i < n8; i += kFThreads) {
    uint32_t p[TC][4];
    load_x_group<TC, LM>(a, tok, 8 * i, vec, x_wrap(a), p);
    if (rms) {
#pragma unroll
      for (int t = 0; t < TC; ++t)
#pragma unroll
        for (int m = 0; m < 4; ++m) p[t][m] = h2_scale(p[t][m], inv[t]);
    }
    store_x_group<TC>(a, smem, 8 * i, p);
  }
}

__device__ __forceinline__ int tc_of(uint32_t nt) { return nt <= 1 ? 1 : (nt <= 2 ? 2 : 4); }
// Interleaved activation rows of an item of nt tokens.
__device__ __forceinline__ int tc_rows(const FusedArgs& a, uint32_t nt) { return tc_of(a.minmax ? 2 * nt : nt); }

template <bool SMALL, int NS, bool DET>
__device__ __forceinline__ void process_dispatch(int tc, const FusedArgs& a, const Chunk& ch, unsigned char* smem,
                                                 const DecBlock& d) {
  if (tc == 1) accumulate<1, SMALL, NS, DET>(a, ch, smem, d);
  else if (tc == 2) accumulate<2, SMALL, NS, DET>(a, ch, smem, d);
  else accumulate<4, SMALL, NS, DET>(a, ch, smem, d);
}

// ------------------------------------------------------------ dense-tile MFMA path
// Heavy experts ([QMoE] "The GPU Decoding Kernel" decodes each weight once;
// with many tokens per expert the multiply is a dense contraction): rows
// [ra, rb) of the item are taken R = mfma_rows at a time.  The tile's
// codewords (row_off[r0] .. row_off[r0 + R]) are decoded by the whole
// workgroup, 16 per thread, with a workgroup prefix of run lengths from the
// position r0 * cols; every nonzero sets a 2-bit code (1: -1, 2: +1) in an LDS
// tile of 16 codes per dword.  Then v_mfma_f32_16x16x32_f16 multiplies 16-row
// tiles of it, expanded to fp16 through a 256-entry table, with 32-column
// slices of the tokens' activations read from global memory; waves split rows
// and K, and partial products meet in fp32 LDS accumulators.  The epilogue is
// the sparse path's.
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

struct MfmaLds {
  uint32_t w, lut, acc, scan, rms, total;   // byte offsets in dynamic LDS, total bytes
};
__host__ __device__ inline MfmaLds mfma_lds(int32_t R, int32_t cols) {
  MfmaLds m;
  const uint32_t wpr = ((uint32_t)cols + 15u) / 16u;
  m.w = 0;
  m.lut = (4u * (uint32_t)R * wpr + 15u) & ~15u;
  m.acc = m.lut + 256u * 8u;
  m.scan = m.acc + 4u * (uint32_t)R * kMfmaMaxTokens;
  m.rms = m.scan + 4u * (kFWaves + 1);
  m.total = m.rms + 4u * kMfmaMaxTokens;
  return m;
}

__device__ __forceinline__ uint32_t div6_exact(uint32_t x) {   // x a multiple of 6
  return (uint32_t)(((uint64_t)x * 0xAAAAAAABull) >> 34);
}

// B fragment of v_mfma_f32_16x16x32_f16: 8 consecutive K of one token
// (with SBM_F_IN_RMS each value is first scaled by the token's 1 / rms and
// rounded to fp16, as the sparse path stages it).
template <bool VEC>
__device__ __forceinline__ half8_t mfma_b_frag(const FusedArgs& a, int32_t tok, int32_t k0, bool rms, float inv) {
  uint4 v = make_uint4(0, 0, 0, 0);
  if (tok >= 0 && k0 < a.cols) {
    const uint16_t* p = a.x + (int64_t)tok * a.cols + k0;
    if (VEC) {
      v = *(const uint4*)p;                      // cols % 8 == 0: k0 + 8 <= cols
    } else {
      uint32_t h[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) h[i] = k0 + i < a.cols ? p[i] : 0u;
      v = make_uint4(h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16);
    }
    if (rms) v = make_uint4(h2_scale(v.x, inv), h2_scale(v.y, inv), h2_scale(v.z, inv), h2_scale(v.w, inv));
  }
  return __builtin_bit_cast(half8_t, v);
}

template <bool VEC>
__device__ __attribute__((noinline)) void mfma_chunk(const FusedArgs& a, unsigned char* smem, const int32_t* perm, const Chunk& ch,
                           uint32_t split7) {
  const int32_t R = a.mfma_rows;
  const uint32_t wpr = ((uint32_t)a.cols + 15u) / 16u;
  const MfmaLds L = mfma_lds(R, a.cols);
  uint32_t* W = (uint32_t*)(smem + L.w);
  uint2* lut = (uint2*)(smem + L.lut);
  float* acc = (float*)(smem + L.acc);
  uint32_t* scan = (uint32_t*)(smem + L.scan);
  float* s_inv = (float*)(smem + L.rms);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int32_t nt = (int32_t)ch.nt;
  const int ntiles = (nt + 15) / 16;
  const bool rms = (a.flags & SBM_F_IN_RMS) != 0;
  wait_vmem_all();        // this wave's part of the image has landed (barriers below)
  if (rms) {
    // 1 / rms of every token row: wave w takes tokens w, w + 8, ...
    for (int32_t t = wave; t < nt; t += kFWaves) {
      const uint16_t* p = a.x + (int64_t)perm[ch.tb + t] * a.cols;
      float ss = 0.f;
      if (VEC) {
        for (int32_t c = 8 * lane; c < a.cols; c += 8 * 64) {
          const uint4 v = *(const uint4*)(p + c);
          ss += h2_ssq(v.x) + h2_ssq(v.y) + h2_ssq(v.z) + h2_ssq(v.w);
        }
      } else {
        for (int32_t c = lane; c < a.cols; c += 64) {
          const float f = (float)__builtin_bit_cast(_Float16, p[c]);
          ss += f * f;
        }
      }
      const float tot = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_incl_scan_f(ss)), 63));
      const float ms = tot / (float)a.cols;
      if (lane == 0) s_inv[t] = ms > 0.f ? 1.0f / sqrtf(ms) : 1.0f;
    }
    __syncthreads();
  }
  for (int b = threadIdx.x; b < 256; b += kFThreads) {
    uint32_t h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t c = (b >> (2 * i)) & 3u;
      h[i] = c == 1u ? 0xBC00u : (c == 2u ? 0x3C00u : 0u);
    }
    lut[b] = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
  }
  // B-fragment tokens of this lane, one per 16-token tile
  int32_t tok[kMfmaMaxTokens / 16];
  float inv[kMfmaMaxTokens / 16];
#pragma unroll
  for (int n = 0; n < kMfmaMaxTokens / 16; ++n) {
    const int32_t t = n * 16 + (lane & 15);
    tok[n] = t < nt ? perm[ch.tb + t] : -1;
    inv[n] = (rms && t < nt) ? s_inv[t] : 1.0f;
  }
  const int nm = R / 16, kparts = kFWaves / nm;
  const int mt = wave % nm, kp = wave / nm;
  const int32_t nks = (a.cols + 31) / 32;
  for (int32_t r0 = ch.ra; r0 < ch.rb; r0 += R) {
    const int32_t Rt = ch.rb - r0 < R ? ch.rb - r0 : R;
    for (uint32_t i = threadIdx.x; i < (uint32_t)R * wpr; i += kFThreads) W[i] = 0u;
    for (uint32_t i = threadIdx.x; i < (uint32_t)R * kMfmaMaxTokens; i += kFThreads) acc[i] = 0.f;
    uint32_t c_lo = a.row_off[ch.off_base + r0], c_hi = a.row_off[ch.off_base + r0 + Rt];
    c_hi = c_hi < ch.n_codes ? c_hi : ch.n_codes;          // offsets are trusted, indexes still bounded
    c_lo = c_lo < c_hi ? c_lo : c_hi;
    __syncthreads();
    // decode: passes of kFThreads * kK codewords
    uint32_t done6 = 0;                        // 6 * columns of the tile decoded by earlier passes
    for (uint32_t cb = c_lo; cb < c_hi; cb += (uint32_t)kFThreads * kK) {
      const uint32_t i0 = cb + threadIdx.x * kK;
      uint32_t sw[kK];
      uint32_t tot = 0;
#pragma unroll
      for (int j = 0; j < kK; ++j) {
        const uint32_t idx = i0 + j;
        const uint32_t c = idx < c_hi ? (uint32_t)a.codes[ch.code_base + idx] : 0u;
        sw[j] = g_tab.tab[table_index(c, split7)] + sign_spread<3>(c, split7);
      }
#pragma unroll
      for (int j = 0; j < kK; ++j) tot += i0 + j < c_hi ? (sw[j] >> 24) : 0u;
      const uint32_t incl = wave_incl_scan(tot);
      if (lane == 63) scan[wave] = incl;
      __syncthreads();
      uint32_t before = 0, all = 0;
#pragma unroll
      for (int w = 0; w < kFWaves; ++w) {
        const uint32_t v = scan[w];
        before += w < wave ? v : 0u;
        all += v;
      }
      uint32_t p6 = a.colsB * (uint32_t)r0 + done6 + before + incl - tot;
#pragma unroll
      for (int j = 0; j < kK; ++j) {
        if (i0 + j < c_hi) {
#pragma unroll
          for (int i = 0; i < 3; ++i) {
            const uint32_t byte = (sw[j] >> (8 * i)) & 0xFFu;
            const uint32_t p6i = 6u * ((byte * 171u) >> 10);          // 6 * position in the run
            const uint32_t k = byte - p6i;                            // 0: -1, 2: +1, 4: zero
            if (k != 4u) {
              const uint32_t q6 = p6 + p6i;
              const uint32_t row = div_magic_dev(q6, a.magic_m, a.magic_s);
              const uint32_t col = div6_exact(q6 - row * a.colsB);
              const int32_t rr = (int32_t)row - r0;
              if (rr >= 0 && rr < Rt)
                atomicOr(&W[(uint32_t)rr * wpr + (col >> 4)], (k == 0u ? 1u : 2u) << ((col & 15u) * 2u));
            }
          }
          p6 += sw[j] >> 24;
        }
      }
      done6 += all;
      __syncthreads();                         // scan reused by the next pass; W complete after the last
    }
    // multiply: wave (mt, kp) takes rows mt*16.. and K-steps kp, kp + kparts, ...
    float4_t cacc[kMfmaMaxTokens / 16];
#pragma unroll
    for (int n = 0; n < kMfmaMaxTokens / 16; ++n) cacc[n] = float4_t{0.f, 0.f, 0.f, 0.f};
    const uint32_t arow = (uint32_t)(mt * 16 + (lane & 15)) * wpr;
    // K-steps in groups of kU: every A and B fragment of a group is requested
    // before its first product, so the global B loads overlap
    constexpr int kU = 4;
    for (int32_t ks0 = kp; ks0 < nks; ks0 += kparts * kU) {
      half8_t A[kU], B[kU][kMfmaMaxTokens / 16];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int32_t k0 = (ks0 + u * kparts) * 32 + 8 * (lane >> 4);
        uint4 av = make_uint4(0, 0, 0, 0);
        if (k0 < a.cols) {
          const uint32_t wv = W[arow + ((uint32_t)k0 >> 4)] >> (((uint32_t)k0 & 15u) * 2u);
          const uint2 lo = lut[wv & 0xFFu], hi = lut[(wv >> 8) & 0xFFu];
          av = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
        A[u] = __builtin_bit_cast(half8_t, av);
#pragma unroll
        for (int n = 0; n < kMfmaMaxTokens / 16; ++n)
          B[u][n] = n < ntiles ? mfma_b_frag<VEC>(a, tok[n], k0, rms, inv[n]) : half8_t{};
      }
#pragma unroll
      for (int u = 0; u < kU; ++u)
#pragma unroll
        for (int n = 0; n < kMfmaMaxTokens / 16; ++n)
          if (n < ntiles) cacc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[u], B[u][n], cacc[n], 0, 0, 0);
    }
    // C layout: lane holds column (token) lane % 16, rows 4 * (lane / 16) + i
#pragma unroll
    for (int n = 0; n < kMfmaMaxTokens / 16; ++n)
      if (n < ntiles) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          atomicAdd(&acc[(mt * 16 + 4 * (lane >> 4) + i) * kMfmaMaxTokens + n * 16 + (lane & 15)], cacc[n][i]);
      }
    __syncthreads();
    for (int32_t i = threadIdx.x; i < Rt * nt; i += kFThreads) {
      const int32_t r = i / nt, t = i - r * nt;
      float v = acc[r * kMfmaMaxTokens + t];
      v *= (float)(*(const _Float16*)(a.scales + ch.scale_base + r0 + r));
      if (a.flags & SBM_F_RELU) v = v > 0.f ? v : 0.f;
      const int64_t o = (int64_t)perm[ch.tb + t] * a.rows + r0 + r;
      if (a.flags & SBM_F_OUT_F32) ((float*)a.y)[o] = v;
      else ((_Float16*)a.y)[o] = (_Float16)v;
    }
    __syncthreads();
  }
}

// Chunks of the current round of a workgroup's slice (LDS) and the block
// sequence counter the waves draw from.
constexpr int kMaxChunks = 16;
__shared__ Chunk s_chunks[kMaxChunks];
__shared__ uint32_t s_nchunks, s_nseq, s_next_seq;
// Rows published per token and not yet counted (layer calls of at most
// kGroupInLds tokens; zero between slices).
__shared__ uint32_t s_pend[kGroupInLds];
__shared__ uint64_t s_gnext;

// Fill the chunk table from global row index g (at most kMaxChunks chunks):
// lane i of wave 0 walks the row arithmetic to chunk i's start, then loads
// its descriptor and row offsets; a wave scan of block counts numbers the
// blocks of the round.
__device__ __forceinline__ void build_chunks(const FusedArgs& a, const uint4* items, uint64_t g, uint64_t g1) {
  static_assert(kMaxChunks <= 64, "one lane per chunk");
  if (tid_v() < 64) {
    const int lane = tid_v();
    uint32_t q = (uint32_t)udiv_small(g + vzero(), (uint32_t)a.rows);
    int32_t ra = (int32_t)(g - (uint64_t)q * a.rows);
    uint64_t gg = g;
    // end row of the chunk starting at row ra of an item, global index gg
    auto chunk_end = [&](int32_t r0, uint64_t at) {
      int64_t e = (int64_t)r0 + a.rmax;
      if (e > a.rows) e = a.rows;
      if ((uint64_t)(e - r0) > g1 - at) e = r0 + (int64_t)(g1 - at);
      return (int32_t)e;
    };
    for (int k = 0; k < lane && gg < g1; ++k) {
      const int32_t e = chunk_end(ra, gg);
      gg += (uint64_t)(e - ra);
      if (e == a.rows) {
        ++q;
        ra = 0;
      } else {
        ra = e;
      }
    }
    const bool exists = lane < kMaxChunks && gg < g1;
    const int32_t rb = exists ? chunk_end(ra, gg) : ra;
    Chunk ch;
    uint32_t nblk = 0;
    if (exists) {
      ch = chunk_at(a, items, q, ra, rb);
      if (ch.ok && ch.b1 >= ch.b0) nblk = ch.b1 - ch.b0 + 1;
    }
    const uint32_t incl = wave_incl_scan(nblk);
    const uint32_t nch = (uint32_t)__popcll(__ballot(exists));
    if (exists) {
      ch.seq0 = incl - nblk;
      s_chunks[lane] = ch;
      if ((uint32_t)lane == nch - 1) {
        s_nseq = incl;
        s_gnext = gg + (uint64_t)(rb - ra);
      }
    }
    if (lane == 0) {
      s_nchunks = nch;
      s_next_seq = 2 * kFWaves;     // blocks 0 .. 2*waves-1 are the waves' first two
      if (nch == 0) {
        s_nseq = 0;
        s_gnext = g1;
      }
    }
  }
  __syncthreads();
}

// Chunk c of the table, every field made wave-uniform (scalar registers).
__device__ __forceinline__ Chunk load_chunk(uint32_t c) {
  const Chunk& m = s_chunks[c];
  auto u32 = [](uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane(v); };
  auto u64 = [&](uint64_t v) { return (uint64_t)u32((uint32_t)v) | ((uint64_t)u32((uint32_t)(v >> 32)) << 32); };
  Chunk ch;
  ch.q = u32(m.q);
  ch.tb = u32(m.tb);
  ch.nt = u32(m.nt);
  ch.ra = (int32_t)u32((uint32_t)m.ra);
  ch.rb = (int32_t)u32((uint32_t)m.rb);
  ch.b0 = u32(m.b0);
  ch.b1 = u32(m.b1);
  ch.code_base = u64(m.code_base);
  ch.n_codes = u32(m.n_codes);
  ch.blk_base = u64(m.blk_base);
  ch.scale_base = u64(m.scale_base);
  ch.off_base = u64(m.off_base);
  ch.seq0 = u32(m.seq0);
  ch.ok = u32((uint32_t)m.ok) != 0;
  ch.mfma = u32((uint32_t)m.mfma) != 0;
  return ch;
}

// Chunk holding block sequence number q (q < s_nseq).
__device__ __forceinline__ uint32_t chunk_of_seq(uint32_t q, uint32_t nch) {
  uint32_t c = 0;
  while (c + 1 < nch && s_chunks[c + 1].seq0 <= q) ++c;
  return c;
}

// Draw the next block for this wave and start loading it.
struct Slot {
  BlockCodes v;
  uint32_t seq;         // 0xFFFFFFFF when empty
};

// first >= 0: take that block sequence number (the waves' first two blocks of
// a round are fixed); otherwise draw the next one from the counter.
// cur, seq_end: the chunk being processed and its end; a block inside it
// needs no chunk-table lookup.
__device__ __forceinline__ Slot grab(const FusedArgs& a, uint32_t nseq, uint32_t nch, int32_t first = -1,
                                     const Chunk* cur = nullptr, uint32_t seq_end = 0) {
  uint32_t q = 0;
  if (first >= 0) {
    q = (uint32_t)first;
  } else {
    if ((threadIdx.x & 63) == 0) q = atomicAdd(&s_next_seq, 1u);
  }
  q = __builtin_amdgcn_readfirstlane(q);   // uniform, so the buffer resources live in scalar registers
  // the same three loads on every path, an empty slot with empty ranges
  uint64_t cb = 0, bb = 0;
  uint32_t nc = 0, b = 0;
  const bool valid = q < nseq;
  if (valid) {
    auto u64 = [](uint64_t v) {
      return (uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)v) |
             ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32)) << 32);
    };
    if (cur && q < seq_end) {       // q >= cur->seq0: the counter only grows
      cb = cur->code_base;
      bb = cur->blk_base;
      nc = cur->n_codes;
      b = cur->b0 + (q - cur->seq0);
    } else {
      const uint32_t c = chunk_of_seq(q, nch);
      cb = u64(s_chunks[c].code_base);
      bb = u64(s_chunks[c].blk_base);
      nc = __builtin_amdgcn_readfirstlane(s_chunks[c].n_codes);
      b = __builtin_amdgcn_readfirstlane(s_chunks[c].b0 + (q - s_chunks[c].seq0));
    }
  }
  Slot sl;
  // the block start is requested with the codes, so that waiting for this
  // block never waits for blocks requested after it
  sl.v = load_block(a, cb, nc, b);
  const __amdgpu_buffer_rsrc_t rb =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.bstart + bb + b), (short)0, valid ? 4 : 0, kBufferFlags);
  sl.v.bst = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rb, 0, 0, 0);
  sl.seq = valid ? q : 0xFFFFFFFFu;
  return sl;
}

// MFMA: the kernel instance that runs dense-tile items (SBM_F_MFMA); the
// default instance has no call in its loop, which keeps its registers unspilled.
template <bool SMALL, bool MFMA, int NS, int LM = 0, bool DET = false>
__device__ __forceinline__ void run_slice(const FusedArgs& a, unsigned char* smem, const int32_t* perm, const uint4* items,
                          uint64_t g0, uint64_t g1, uint32_t split7) {
  // the image copy issued at kernel entry is waited for just before the
  // barrier that follows the first activation staging (or inside the first
  // dense tile), so the chunk table and first blocks are fetched meanwhile
  racc_clear<DET>(a, smem);
  build_chunks(a, items, g0, g1);
  uint32_t cur_q = 0xFFFFFFFFu;
  while (true) {
    const uint32_t nch = __builtin_amdgcn_readfirstlane(s_nchunks), nseq = __builtin_amdgcn_readfirstlane(s_nseq);
    if (nch == 0) break;
    // Two blocks in flight per wave: A is decoded next, then B.  A block's
    // slot is refilled as soon as its codes are decoded, and the loop is
    // unrolled over A and B, so no slot is copied (a copy would wait for the
    // loads still landing in it).
    const int32_t wave = (int32_t)(tid_v() >> 6);
    Slot A = grab(a, nseq, nch, wave), B = grab(a, nseq, nch, wave + kFWaves);
    for (uint32_t c = 0; c < nch; ++c) {
      const Chunk ch = load_chunk(c);
      if (MFMA && ch.mfma) {
        // dense tiles overwrite the accumulators and the staged activations
        if (ch.ok) {
          if (x_vec(a)) mfma_chunk<true>(a, smem, perm, ch, split7);
          else mfma_chunk<false>(a, smem, perm, ch, split7);
        }
        racc_clear<DET>(a, smem);
        cur_q = 0xFFFFFFFFu;
        __syncthreads();
        continue;
      }
      const int tc = tc_rows(a, ch.nt);
      if (ch.q != cur_q) {
        if (tc == 1) stage_x<1, LM>(a, smem, perm, ch.tb, ch.nt);
        else if (tc == 2) stage_x<2, LM>(a, smem, perm, ch.tb, ch.nt);
        else stage_x<4, LM>(a, smem, perm, ch.tb, ch.nt);
        cur_q = ch.q;
        wait_vmem_all();      // this wave's part of the image has landed
        __syncthreads();
      }
      const uint32_t seq_end = c + 1 < nch ? __builtin_amdgcn_readfirstlane(s_chunks[c + 1].seq0) : nseq;
      auto step = [&](Slot& sl) {
        if (sl.seq >= seq_end) return false;
        DecBlock d;
        decode_block<NS>(sl.v, split7, d);
        sl = grab(a, nseq, nch, -1, &ch, seq_end);
        process_dispatch<SMALL, NS, DET>(tc, a, ch, smem, d);
        return true;
      };
      while (step(A)) {
        if (!step(B)) {           // B's block starts the next chunk: it goes first
          const Slot t = A;
          A = B;
          B = t;
          break;
        }
      }
      // This wave has no more blocks of the chunk.  While the others finish,
      // request the row scales of this thread's epilogue rows and, when the
      // next chunk starts another item, that item's activations.
      const int32_t R = ch.rb - ch.ra;
      uint32_t sc[kEpiRegs];
#pragma unroll
      for (int k = 0; k < kEpiRegs; ++k) {
        const int32_t i = (int32_t)tid_v() + k * kFThreads;   // accumulator slot, row i - 1
        const bool live = ch.ok && i >= 1 && i <= R;
        if (a.minmax)     // (w_min, w_max) of the row, one dword
          sc[k] = live ? ((const uint32_t*)a.scales)[ch.scale_base / 2 + ch.ra + i - 1] : 0u;
        else
          sc[k] = live ? a.scales[ch.scale_base + ch.ra + i - 1] : 0u;
      }
      bool next_new = false, next_pre = false;
      Chunk nx;
      XPre xp;
      if (c + 1 < nch) {
        nx = load_chunk(c + 1);
        next_new = nx.q != ch.q && !nx.mfma;
        const int ntc = tc_rows(a, nx.nt);
        if (next_new && x_prefetchable(a, ntc)) {
          next_pre = true;
          wait_tokens<LM>(a, perm, nx.tb, nx.nt);
          if (ntc == 1) xpre_load<1, LM>(a, perm, nx.tb, nx.nt, xp);
          else if (ntc == 2) xpre_load<2, LM>(a, perm, nx.tb, nx.nt, xp);
          else xpre_load<4, LM>(a, perm, nx.tb, nx.nt, xp);
        }
      }
      __syncthreads();
      // epilogue: scale, activation, convert, scatter to token order; the
      // accumulator slots [0, R + 1] of tokens t < tc are cleared for the next chunk
#pragma unroll
      for (int k = 0; k < kEpiRegs; ++k) {
        const int32_t i = (int32_t)tid_v() + k * kFThreads;
        if (i < R + 2 && a.minmax) {
          // y = w_min * S1 + w_max * S2 = ((w_max - w_min) * A + (w_max + w_min) * B) / 2
          const float wmin = (float)__builtin_bit_cast(_Float16, (uint16_t)(sc[k] & 0xFFFFu));
          const float wmax = (float)__builtin_bit_cast(_Float16, (uint16_t)(sc[k] >> 16));
          for (int u = 0; 2 * u < tc; ++u) {
            const float A = racc_take<DET>(a, smem, 2 * u, i), B = racc_take<DET>(a, smem, 2 * u + 1, i);
            if (ch.ok && i >= 1 && i <= R && (uint32_t)u < ch.nt) {
              float v = 0.5f * ((wmax - wmin) * A + (wmax + wmin) * B);
              if (a.flags & SBM_F_RELU) v = v > 0.f ? v : 0.f;
              const int64_t o = (int64_t)perm[ch.tb + u] * a.rows + ch.ra + i - 1;
              if (a.flags & SBM_F_OUT_F32) ((float*)a.y)[o] = v;
              else ((_Float16*)a.y)[o] = (_Float16)v;
            }
          }
        } else if (i < R + 2) {
          const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)sc[k]);
          for (int t = 0; t < tc; ++t) {
            float v = racc_take<DET>(a, smem, t, i);
            if (ch.ok && i >= 1 && i <= R && (uint32_t)t < ch.nt) {
              v *= s;
              if (a.flags & SBM_F_RELU) v = v > 0.f ? v : 0.f;
              const int64_t o = (int64_t)perm[ch.tb + t] * a.rows + ch.ra + i - 1;
              if (lm_out<LM>(a)) {   // read by the next phase: written through to device scope
                __hip_atomic_store((uint16_t*)a.y + o, __builtin_bit_cast(uint16_t, (_Float16)v), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
              } else if (a.flags & SBM_F_OUT_F32) {
                ((float*)a.y)[o] = v;
              } else {
                ((_Float16*)a.y)[o] = (_Float16)v;
              }
            }
          }
        }
      }
      if (next_new) {
        const int ntc = tc_rows(a, nx.nt);
        if (next_pre) {
          if (ntc == 1) xpre_store<1>(a, smem, xp);
          else if (ntc == 2) xpre_store<2>(a, smem, xp);
          else xpre_store<4>(a, smem, xp);
        } else {
          if (ntc == 1) stage_x<1, LM>(a, smem, perm, nx.tb, nx.nt);
          else if (ntc == 2) stage_x<2, LM>(a, smem, perm, nx.tb, nx.nt);
          else stage_x<4, LM>(a, smem, perm, nx.tb, nx.nt);
        }
        cur_q = nx.q;
      }
      // Published rows: with at most kGroupInLds tokens their per-token counts
      // are gathered in LDS and raised once, at the end of the slice, after a
      // single wait for the stores (a wait per chunk would hold up the next
      // chunk's blocks); otherwise raised here, once the chunk's rows are stored.
      const bool pub = lm_out<LM>(a), pend = pub && a.n_tokens <= kGroupInLds;
      if (pub && !pend) wait_vmem_all();   // this thread's output rows have reached device scope
      __syncthreads();
      if (pub) {
        // every row of the chunk is written: raise its tokens' counts (also
        // for a refused expert, whose rows stay unwritten, so no wait hangs)
        if (tid_v() < ch.nt) {
          const int32_t t = perm[ch.tb + tid_v()];
          if (pend) s_pend[t] += (uint32_t)(ch.rb - ch.ra);     // one thread per token of the chunk
          else __hip_atomic_fetch_add(a.tok_done + t, (uint32_t)(ch.rb - ch.ra), __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    const uint64_t gn = s_gnext;
    __syncthreads();      // every wave has read the table before it is rebuilt
    if (gn >= g1) break;
    build_chunks(a, items, gn, g1);
  }
  if (lm_out<LM>(a) && a.n_tokens <= kGroupInLds) {
    wait_vmem_all();      // every output row of the slice has reached device scope
    __syncthreads();
    for (int32_t t = tid_v(); t < a.n_tokens; t += kFThreads) {
      const uint32_t n = s_pend[t];
      if (n) {
        __hip_atomic_fetch_add(a.tok_done + t, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_pend[t] = 0;
      }
    }
  }
}

// Token grouping inside the fused kernel for n_tokens <= kGroupInLds: every
// workgroup derives the same items as group_kernel from the ids alone.  The
// sort key (expert << 8 | token) is unique; a token's rank among the keys is
// its place in perm, and rank minus the count of smaller experts its place in
// its expert's run.  Items start at run places divisible by tcmax; a wave
// scan over sorted places numbers them and sums their weights.
__shared__ uint4 s_items[kGroupInLds];
__shared__ int32_t s_perm[kGroupInLds];
__shared__ uint32_t s_ghdr[4];   // n_items, total weight, valid tokens, bad descriptors
__shared__ uint64_t s_slice[2];  // this workgroup's [g0, g1)
constexpr uint32_t kGroupScratch = 6 * kGroupInLds * 4;   // bytes of dynamic LDS used while grouping
static_assert(kFThreads % kGroupInLds == 0 && kGroupInLds == 128, "4 threads per token, 2 places per lane");

__device__ __forceinline__ void group_lds(const FusedArgs& a, uint32_t* sc, int32_t my_id) {
  constexpr int N = kGroupInLds;
  constexpr int kParts = kFThreads / N;
  constexpr uint32_t kNone = 0xFFFFFFFFu;
  uint32_t* keys = sc;           // by token
  uint32_t* rk = sc + N;         // rank, smaller experts, same expert: by token
  uint32_t* lt = sc + 2 * N;
  uint32_t* eq = sc + 3 * N;
  uint32_t* nts = sc + 4 * N;    // item size at an item's first sorted place, else 0
  uint32_t* ks = sc + 5 * N;     // key by sorted place
  const int32_t T = a.n_tokens;
  const int tid = tid_v();
  if (tid < N) {
    uint32_t key = kNone;
    if (tid < T && my_id >= 0 && my_id < a.n_experts) key = ((uint32_t)my_id << 8) | (uint32_t)tid;
    keys[tid] = key;
    rk[tid] = 0;
    lt[tid] = 0;
    eq[tid] = 0;
    nts[tid] = 0;
    if (tid < 4) s_ghdr[tid] = 0;
  }
  __syncthreads();
  {
    const int t = tid % N, part = tid / N;
    const int span = ((T + 4 * kParts - 1) / (4 * kParts)) * 4;   // keys per part, multiple of 4
    const uint32_t key = t < T ? keys[t] : kNone;
    if (key != kNone) {
      const uint32_t ek = key >> 8;
      uint32_t r = 0, l = 0, m = 0;
      const int j0 = part * span, j1 = j0 + span < N ? j0 + span : N;
      for (int j = j0; j < j1; j += 4) {
        const uint4 k4 = *(const uint4*)(keys + j);
        const uint32_t kk[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          r += kk[u] < key;
          l += (kk[u] >> 8) < ek;
          m += (kk[u] >> 8) == ek;
        }
      }
      if (r) atomicAdd(&rk[t], r);
      if (l) atomicAdd(&lt[t], l);
      atomicAdd(&eq[t], m);
    }
  }
  __syncthreads();
  if (tid < N) {
    const uint32_t key = keys[tid];
    const bool valid = key != kNone;
    if (valid) {
      const uint32_t rank = rk[tid], off = rank - lt[tid], cnt = eq[tid];
      const bool heavy = a.mfma_rows > 0 && cnt >= (uint32_t)kMfmaMinTokens;
      const uint32_t span = heavy ? (uint32_t)kMfmaMaxTokens : (uint32_t)a.titem;
      s_perm[rank] = tid;
      ks[rank] = key;
      if (off % span == 0) nts[rank] = (cnt - off < span ? cnt - off : span) | (heavy ? kItemMfma : 0u);
    }
    const uint64_t b = __ballot(valid);
    if ((tid & 63) == 0 && b) atomicAdd(&s_ghdr[2], (uint32_t)__popcll(b));
  }
  __syncthreads();
  if (tid < 64) {
    const uint32_t n0 = nts[2 * tid], n1 = nts[2 * tid + 1];
    const uint32_t w0 = n0 ? item_weight(n0, a.minmax) : 0u, w1 = n1 ? item_weight(n1, a.minmax) : 0u;
    const uint32_t c = (n0 != 0) + (n1 != 0);
    const uint32_t ci = wave_incl_scan(c), wi = wave_incl_scan(w0 + w1);
    uint32_t q = ci - c, wp = wi - w0 - w1;
    if (n0) {
      s_items[q] = make_uint4(ks[2 * tid] >> 8, 2 * tid, n0, wp);
      ++q;
      wp += w0;
    }
    if (n1) s_items[q] = make_uint4(ks[2 * tid + 1] >> 8, 2 * tid + 1, n1, wp);
    if (tid == 63) {
      s_ghdr[0] = ci;
      s_ghdr[1] = wi;
    }
    // this workgroup's slice: weighted positions u0, u1 of the (item, row)
    // space; item q covers [wpre_q * rows, (wpre_q + w_q) * rows), each of
    // its rows weighing w_q (the same split as group_kernel's)
    const uint32_t n_items = __builtin_amdgcn_readlane(ci, 63), wtot = __builtin_amdgcn_readlane(wi, 63);
    const uint32_t F = a.item_cost;
    const uint64_t rows = (uint64_t)a.rows, wall = (uint64_t)wtot * rows + (uint64_t)n_items * F;
    const uint32_t sl = xcd_slice(blockIdx.x, (uint32_t)a.grid);
    const uint64_t u[2] = {slice_div(wall * sl, (uint32_t)a.grid), slice_div(wall * (sl + 1), (uint32_t)a.grid)};
    uint32_t qi = ci - c, wq = wi - w0 - w1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t nh = h ? n1 : n0, wh = h ? w1 : w0;
      if (nh) {
        const uint64_t pq = (uint64_t)wq * rows + (uint64_t)qi * F;
#pragma unroll
        for (int k = 0; k < 2; ++k)
          if (u[k] >= pq && u[k] < pq + F + (uint64_t)wh * rows) s_slice[k] = boundary_in_item(u[k], pq, qi, wh, F, rows);
        ++qi;
        wq += wh;
      }
    }
    if (tid == 0) {
#pragma unroll
      for (int k = 0; k < 2; ++k)
        if (u[k] >= wall) s_slice[k] = (uint64_t)n_items * rows;
    }
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    // descriptors of the touched experts; workgroup 0 alone writes the error word
    const uint32_t n_items = s_ghdr[0];
    for (uint32_t q = tid_v(); q < n_items; q += kFThreads)
      if (const uint32_t err = desc_err(a.experts[s_items[q].x], a.rows, a.cols, a.minmax, image_tag(a)))
        atomicOr(&s_ghdr[3], err);
    __syncthreads();
    if (tid_v() == 0) a.ws[0] = (((uint32_t)T - s_ghdr[2]) & kErrCountMask) | s_ghdr[3];
  }
}

// Token grouping for n_tokens <= 64 by wave 0 alone, with no workgroup
// barrier until the results are published: lane t holds token t's key
// (expert << 6 | t); its rank among the keys (a count over all 64 keys, read
// back from LDS as broadcasts) is its place in perm.  Lane r then reads the
// r-th smallest key back;
// expert runs and item starts are ballots over the sorted keys, item numbers
// are prefix popcounts and item weights a wave scan.  Items, perm and the
// workgroup's slice are the same as group_lds derives.
__device__ __forceinline__ void group_wave(const FusedArgs& a, uint32_t* sc, int32_t my_id) {
  constexpr uint32_t kNone = 0x7FFFFFFFu;   // above every valid key (< 2^30)
  const int32_t T = a.n_tokens;
  if (tid_v() < 64) {
    const uint32_t lane = tid_v();
    const bool valid = (int32_t)lane < T && my_id >= 0 && my_id < a.n_experts;
    const uint32_t key = valid ? (((uint32_t)my_id << 6) | lane) : kNone;
    uint32_t* ks = sc + 64;                 // keys by lane, then by sorted place
    sc[lane] = key;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // keys are below 2^31, so the sign bit of kk - key is [kk < key]
    uint32_t rk[4] = {0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < 64; u += 4) {       // every lane reads the same words
      const uint4 k4 = *(const uint4*)(sc + u);
      rk[0] += (k4.x - key) >> 31;
      rk[1] += (k4.y - key) >> 31;
      rk[2] += (k4.z - key) >> 31;
      rk[3] += (k4.w - key) >> 31;
    }
    const uint32_t rank = rk[0] + rk[1] + rk[2] + rk[3];
    const uint32_t nv = (uint32_t)__popcll(__ballot(valid));
    if (valid) ks[rank] = key;              // valid keys rank below every kNone
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint32_t r = lane;
    const bool in = r < nv;
    const uint32_t k = in ? ks[r] : kNone;
    const uint32_t kp = (in && r > 0) ? ks[r - 1] : kNone;
    const uint32_t e = k >> 6;
    const bool start = in && (r == 0 || (kp >> 6) != e);
    const uint64_t sb = __ballot(start);
    const uint64_t upto = ((uint64_t)2 << r) - 1;      // bits 0..r (r = 63: all)
    const uint64_t below = sb & upto, above = sb & ~upto;
    const uint32_t rs = below ? 63u - (uint32_t)__builtin_clzll(below) : 0u;   // this run's first place
    const uint32_t re = above ? (uint32_t)__builtin_ctzll(above) : nv;   // next run's first place
    const uint32_t off = r - rs, cnt = re - rs;
    const bool heavy = a.mfma_rows > 0 && cnt >= (uint32_t)kMfmaMinTokens;
    const uint32_t span = heavy ? (uint32_t)kMfmaMaxTokens : (uint32_t)a.titem;
    const bool istart = in && off % span == 0;
    const uint32_t nt = istart ? ((cnt - off < span ? cnt - off : span) | (heavy ? kItemMfma : 0u)) : 0u;
    const uint64_t ib = __ballot(istart);
    const uint32_t q = (uint32_t)__popcll(ib & (((uint64_t)1 << r) - 1));
    const uint32_t w = istart ? item_weight(nt, a.minmax) : 0u;
    const uint32_t wi = wave_incl_scan(w);
    const uint32_t wq = wi - w;
    if (in) s_perm[r] = (int32_t)(k & 63u);
    if (istart) s_items[q] = make_uint4(e, r, nt, wq);

    const uint32_t n_items = (uint32_t)__popcll(ib), wtot = __builtin_amdgcn_readlane(wi, 63);
    // this workgroup's slice [u0, u1) of the weighted (item, row) space
    const uint32_t F = a.item_cost;
    const uint64_t rows = (uint64_t)a.rows, wall = (uint64_t)wtot * rows + (uint64_t)n_items * F;
    // lane h computes u_h, then both are broadcast
    const uint64_t uh = slice_div(wall * (xcd_slice(blockIdx.x, (uint32_t)a.grid) + (lane & 1u) + vzero()),
                                  (uint32_t)a.grid);
    const uint64_t u[2] = {
        (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)uh, 0) |
            ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(uh >> 32), 0) << 32),
        (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)uh, 1) |
            ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(uh >> 32), 1) << 32)};
    if (istart) {
      const uint64_t pq = (uint64_t)wq * rows + (uint64_t)q * F;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        if (u[h] >= pq && u[h] < pq + F + (uint64_t)w * rows) s_slice[h] = boundary_in_item(u[h], pq, q, w, F, rows);
    }
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        if (u[h] >= wall) s_slice[h] = (uint64_t)n_items * rows;
      s_ghdr[0] = n_items;
      s_ghdr[1] = wtot;
      s_ghdr[2] = nv;
      s_ghdr[3] = 0;
    }
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    // descriptors of the touched experts; workgroup 0 alone writes the error word
    const uint32_t n_items = s_ghdr[0];
    for (uint32_t q = tid_v(); q < n_items; q += kFThreads)
      if (const uint32_t err = desc_err(a.experts[s_items[q].x], a.rows, a.cols, a.minmax, image_tag(a)))
        atomicOr(&s_ghdr[3], err);
    __syncthreads();
    if (tid_v() == 0) a.ws[0] = (((uint32_t)T - s_ghdr[2]) & kErrCountMask) | s_ghdr[3];
  }
}

// Instances: MODE 0 the sparse path, 1 with dense-tile MFMA items, 2 with the
// per-row min/max grid; 3 and 4 are 0 and 2 with the 4-slot decode image;
// 5 to 8 are 0, 2, 3 and 4 with fixed-point row accumulators
// (SBM_F_DETERMINISTIC).  The grid flag is made a constant of each instance,
// so the default instance carries none of its code.
constexpr int kModes = 9;
__host__ __device__ constexpr int mode_base(int m) { return m == 5 ? 0 : m == 6 ? 2 : m == 7 ? 3 : m == 8 ? 4 : m; }
__host__ __device__ constexpr int mode_slots(int m) { return mode_base(m) >= 3 ? 4 : 3; }
template <int MODE>
__global__ __launch_bounds__(kFThreads) void fused_kernel(FusedArgs a) {
  constexpr int BASE = mode_base(MODE);
  constexpr bool DET = MODE >= 5;
  constexpr bool MFMA = BASE == 1;
  constexpr int NS = mode_slots(MODE);
  a.minmax = (BASE == 2 || BASE == 4) ? 1 : 0;
  extern __shared__ __align__(16) unsigned char smem[];
  // Requests in order of need: token ids (every thread, no branch, so the
  // request goes out with the first argument loads), the image header in one
  // scalar load, then the decode image (stored to LDS once the slice is
  // known), so waiting for the ids never waits for the image.
  const int32_t tq = (int32_t)threadIdx.x < a.n_tokens ? (int32_t)threadIdx.x : a.n_tokens - 1;
  const int32_t my_id = a.ids[tq];
  const uint4 hdr = *(const uint4*)a.image;       // magic, version, split, n_tab
  stage_tables_dma<NS>(a.image);
  // the table indexes stay below n_tab <= the table's capacity for every codeword
  const bool image_ok = hdr.x == kImageMagic && hdr.y == (NS == 3 ? kImageVersion : kImage4Version) &&
                        hdr.z <= SBM_DICT_ENTRIES && hdr.w == hdr.z + (SBM_DICT_ENTRIES - hdr.z + 7u) / 8u &&
                        hdr.w <= (NS == 3 ? kTabEntries : kTab4Entries);
  const uint32_t split7 = 7u * hdr.z;
  const int32_t* perm;
  const uint4* items;
  uint64_t g0, g1;
  if (a.group_in_lds) {
    if (a.n_tokens <= 64) group_wave(a, (uint32_t*)smem, my_id);
    else group_lds(a, (uint32_t*)smem, (int32_t)threadIdx.x < a.n_tokens ? my_id : -1);
    if (!image_ok) {
      // the same thread wrote the grouping's word: keep its id count and shape
      // bit; the dictionary comparison was made against a damaged header
      if (blockIdx.x == 0 && threadIdx.x == 0) {
        a.ws[0] = (a.ws[0] & ~kErrDict) | kErrBadImage;
        if (a.err_out) *a.err_out = a.ws[0];
      }
      return;               // (s_endpgm waits for the table copy still in flight, as on an empty slice)
    }
    if (a.err_out && blockIdx.x == 0 && threadIdx.x == 0) *a.err_out = a.ws[0];   // this thread wrote it
    g0 = s_slice[0];
    g1 = s_slice[1];
    perm = s_perm;
    items = s_items;
  } else {
    if (!image_ok) {   // group_kernel's word is complete (stream order); its dictionary bit is void
      if (blockIdx.x == 0 && threadIdx.x == 0) {
        a.ws[0] = (a.ws[0] & ~kErrDict) | kErrBadImage;
        if (a.err_out) *a.err_out = a.ws[0];
      }
      return;
    }
    if (a.err_out && blockIdx.x == 0 && threadIdx.x == 0) *a.err_out = a.ws[0];
    const WsLayout L = ws_layout(a.n_experts, a.n_tokens);
    const uint64_t* bounds = (const uint64_t*)(a.ws + L.bounds);
    const uint32_t sl = xcd_slice(blockIdx.x, (uint32_t)a.grid);
    g0 = bounds[sl];
    g1 = bounds[sl + 1];
    perm = (const int32_t*)(a.ws + L.perm);
    items = (const uint4*)(a.ws + L.items);
  }
  if (g0 >= g1) return;
  if (a.cols < kSmallCols) run_slice<true, MFMA, NS, 0, DET>(a, smem, perm, items, g0, g1, split7);
  else run_slice<false, MFMA, NS, 0, DET>(a, smem, perm, items, g0, g1, split7);
}

// ------------------------------------------------------------ layer calls
// Several projections in one launch ([QMoE] "The GPU Decoding Kernel": the
// experts are FFNs whose two matrices are multiplied in turn, layer after
// layer).  Phase p is layer p / 2's up projection (ReLU) when p is even, its
// down projection when p is odd; a layer's up phase reads the previous
// layer's output scaled to unit RMS per token (the glue between layers).
// Every workgroup runs its slice of each phase in turn.  A phase's tokens are
// grouped, its chunk table is built and its first code blocks are requested
// as soon as the workgroup has finished the previous phase; only the staging
// of a token's activations waits, until every input row of that token is
// written (per-token counts raised by the previous phase's chunks, rows
// written and read coherently at device scope, so no cache-wide writeback or
// invalidation is needed).  A workgroup's next slice covers about the same
// experts as its last one, so it mostly waits for its neighbours, not for the
// slowest workgroup of the launch.  All workgroups are resident (one per CU,
// at most the CU count), and every wait is bounded.
// Sync area at the start of the layer workspace (uint32 words): [0] the
// finished call's error word, [1] the running error word, [2] workgroups
// done, [16 ..) one count per token and phase (all phases but the last).
// The last workgroup to finish publishes the error word and clears the rest,
// so a call leaves the area ready for the next one (the caller zeroes it
// once, before the first call).
constexpr uint32_t kSyncHdr = 16;
constexpr int kMaxLayers = 32;
struct LayerProj {
  const uint16_t* codes;
  const uint32_t* row_off;
  const uint32_t* bstart;
  const uint16_t* scales;
  const sbm_matrix_desc* experts;
};
struct LayerTab {
  LayerProj up[kMaxLayers], dn[kMaxLayers];
  uint16_t* h;            // [n_layers][T][up rows]: every layer's h
  uint16_t* y;            // [n_layers][T][down rows]: every layer's output (the input of the next)
  uint32_t ws_words;      // words of workspace per phase (grouping state)
  int32_t n_layers;
};
static_assert(2 * sizeof(FusedArgs) + sizeof(LayerTab) + sizeof(void*) <= 4096, "kernel arguments within 4 KB");
__shared__ uint32_t s_last;

// Arguments of phase p from the up and down templates (which hold layer 0's
// arrays and the shape, plan, flags and buffers of every layer).
__device__ __forceinline__ FusedArgs phase_args(const FusedArgs& up, const FusedArgs& dn, const LayerTab& tab, int p,
                                                uint32_t* sync) {
  const int l = p >> 1, n_ph = 2 * tab.n_layers;
  const bool is_up = (p & 1) == 0;
  FusedArgs a = is_up ? up : dn;
  const LayerProj& lp = is_up ? tab.up[l] : tab.dn[l];
  a.codes = lp.codes;
  a.row_off = lp.row_off;
  a.bstart = lp.bstart;
  a.scales = lp.scales;
  a.experts = lp.experts;
  a.ids = up.ids + (int64_t)l * up.n_tokens;
  a.ws = up.ws + (uint64_t)p * tab.ws_words;
  const uint64_t hl = (uint64_t)l * (uint64_t)up.n_tokens * (uint64_t)up.rows;    // layer l's h
  const uint64_t yl = (uint64_t)l * (uint64_t)up.n_tokens * (uint64_t)dn.rows;    // layer l's output
  if (is_up) {
    a.y = tab.h + hl;
    if (l > 0) {
      a.x = tab.y + (yl - (uint64_t)up.n_tokens * (uint64_t)dn.rows);
      a.flags = (a.flags & ~SBM_F_IN_BF16) | SBM_F_IN_RMS;
      a.x_bytes = (uint32_t)((uint64_t)a.n_tokens * (uint64_t)a.cols * 2u);
    }
  } else {
    a.x = tab.h + hl;
    a.y = tab.y + yl;
  }
  a.lm = (p + 1 < n_ph ? 1u : 0u) | (p > 0 ? 2u : 0u);
  a.tok_done = sync + kSyncHdr + (uint64_t)p * (uint64_t)a.n_tokens;
  a.tok_wait = sync + kSyncHdr + (uint64_t)(p > 0 ? p - 1 : 0) * (uint64_t)a.n_tokens;
  a.tok_expect = (uint32_t)(is_up ? dn.rows : up.rows);
  return a;
}

// One phase: group the tokens (in LDS, or read the grouping launch's result),
// then run this workgroup's slice.
// Expert ids of the current and the next layer, by token (in-LDS grouping).
__shared__ int32_t s_ids[2][kGroupInLds];

__device__ __forceinline__ void stack_phase(const FusedArgs& a, int p, unsigned char* smem, bool image_ok,
                                            uint32_t split7, uint32_t* sync, int32_t n_layers) {
  const int32_t* perm;
  const uint4* items;
  uint64_t g0, g1;
  const int32_t l = p >> 1;
  if (a.group_in_lds) {
    const int32_t t = (int32_t)tid_v();
    const int32_t my_id = t < a.n_tokens ? s_ids[l & 1][t] : -1;
    // an up phase requests the next layer's ids, stored once the grouping is done
    const bool fetch = (p & 1) == 0 && l + 1 < n_layers && t < a.n_tokens;
    const int32_t next_id = fetch ? a.ids[a.n_tokens + t] : 0;
    if (a.n_tokens <= 64) group_wave(a, (uint32_t*)smem, my_id);
    else group_lds(a, (uint32_t*)smem, my_id);
    if (fetch) s_ids[(l + 1) & 1][t] = next_id;     // the other layer's slot, read after later barriers
    g0 = s_slice[0];
    g1 = s_slice[1];
    perm = s_perm;
    items = s_items;
  } else {
    // the grouping launch cut the phase into a.grid slices; the layer launch
    // may hold more workgroups (another phase's count)
    const WsLayout L = ws_layout(a.n_experts, a.n_tokens);
    const uint64_t* bounds = (const uint64_t*)(a.ws + L.bounds);
    const bool mine = (int32_t)blockIdx.x < a.grid;
    const uint32_t sl = mine ? xcd_slice(blockIdx.x, (uint32_t)a.grid) : 0u;
    g0 = mine ? bounds[sl] : 0;
    g1 = mine ? bounds[sl + 1] : 0;
    perm = (const int32_t*)(a.ws + L.perm);
    items = (const uint4*)(a.ws + L.items);
  }
  if (blockIdx.x == 0 && tid_v() == 0) {
    // this thread wrote (or the grouping kernel before this launch wrote) the
    // phase's word: invalid ids counted once per layer, the flag bits of all phases
    uint32_t w = a.ws[0];
    if (p & 1) w &= ~kErrCountMask;
    if (!image_ok) w = (w & ~kErrDict) | kErrBadImage;
    if (w) __hip_atomic_fetch_or(sync + 1, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (blockIdx.x == 0 && image_ok && lm_out<3>(a)) {
    // a token whose expert id is out of range gets no rows in this layer:
    // its count is raised at once, so the next phase does not wait for it
    // (its output is invalid, and the error word counts it)
    for (int32_t t = tid_v(); t < a.n_tokens; t += kFThreads) {
      const int32_t e = a.ids[t];
      if (e < 0 || e >= a.n_experts)
        __hip_atomic_fetch_add(a.tok_done + t, (uint32_t)a.rows, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (image_ok && g0 < g1) run_slice<false, false, 3, 3>(a, smem, perm, items, g0, g1, split7);
  __syncthreads();      // the grouping's LDS is rebuilt by the next phase
}

template <int DUMMY>
__global__ __launch_bounds__(kFThreads) void stack_kernel(const FusedArgs up, const FusedArgs dn, const LayerTab tab,
                                                          uint32_t* sync) {
  extern __shared__ __align__(16) unsigned char smem[];
  if (up.group_in_lds && (int32_t)tid_v() < up.n_tokens) s_ids[0][tid_v()] = up.ids[tid_v()];
  const uint4 hdr = *(const uint4*)up.image;
  stage_tables_dma<3>(up.image);
  const bool image_ok = hdr.x == kImageMagic && hdr.y == kImageVersion && hdr.z <= SBM_DICT_ENTRIES &&
                        hdr.w == hdr.z + (SBM_DICT_ENTRIES - hdr.z + 7u) / 8u && hdr.w <= kTabEntries;
  const uint32_t split7 = 7u * hdr.z;
  for (int32_t t = tid_v(); t < kGroupInLds; t += kFThreads) s_pend[t] = 0;   // read after the grouping's barriers
  for (int p = 0; p < 2 * tab.n_layers; ++p) {
    const FusedArgs a = phase_args(up, dn, tab, p, sync);
    stack_phase(a, p, smem, image_ok, split7, sync, tab.n_layers);
  }
  wait_vmem_all();        // every store and count of this workgroup is complete
  __syncthreads();
  if (tid_v() == 0)
    s_last = __hip_atomic_fetch_add(sync + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1;
  __syncthreads();
  if (s_last) {
    // the other workgroups are done: publish the error word, clear the counts
    const int32_t n_cnt = (2 * tab.n_layers - 1) * up.n_tokens;
    for (int32_t t = tid_v(); t < n_cnt; t += kFThreads)
      __hip_atomic_store(sync + kSyncHdr + t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid_v() == 0) {
      const uint32_t err = __hip_atomic_load(sync + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(sync, err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(sync + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(sync + 2, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Layer calls of more than kGroupInLds tokens: workgroup p groups phase p into
// its part of the workspace (the tables group_kernel writes), one launch for
// every phase of the call.
__global__ __launch_bounds__(kThreads) void stack_group_kernel(const FusedArgs up, const FusedArgs dn,
                                                               const LayerTab tab, uint32_t* sync) {
  const FusedArgs a = phase_args(up, dn, tab, (int)blockIdx.x, sync);
  group_body(a.ids, a.n_tokens, a.n_experts, a.titem, a.rows, a.cols, a.grid, a.item_cost, 0, a.minmax, a.experts,
             a.image, a.ws);
}

// Layer calls of several layers and at most kGroupInLds tokens: workgroup p
// groups phase p in LDS (as the projection kernel does) and writes the tables
// the layer launch then reads from the workspace (token order, items, the
// bounds of every slice), so no workgroup of the layer launch groups.
__global__ __launch_bounds__(kFThreads) void stack_plan_kernel(const FusedArgs up, const FusedArgs dn,
                                                              const LayerTab tab, uint32_t* sync) {
  extern __shared__ __align__(16) unsigned char smem[];
  const FusedArgs a = phase_args(up, dn, tab, (int)blockIdx.x, sync);
  const int32_t t = (int32_t)tid_v();
  const int32_t my_id = t < a.n_tokens ? a.ids[t] : -1;
  if (a.n_tokens <= 64) group_wave(a, (uint32_t*)smem, my_id);
  else group_lds(a, (uint32_t*)smem, my_id);
  __syncthreads();
  const uint32_t n_items = s_ghdr[0], wtot = s_ghdr[1];
  // the phase's error word (the grouping writes it in workgroup 0 only):
  // tokens with an id out of range, descriptors that disagree with the call
  for (uint32_t q = (uint32_t)t; q < n_items; q += kFThreads)
    if (const uint32_t err = desc_err(a.experts[s_items[q].x], a.rows, a.cols, a.minmax, image_tag(a)))
      atomicOr(&s_ghdr[3], err);
  __syncthreads();
  if (t == 0) a.ws[0] = (((uint32_t)a.n_tokens - s_ghdr[2]) & kErrCountMask) | s_ghdr[3];
  const WsLayout L = ws_layout(a.n_experts, a.n_tokens);
  int32_t* perm = (int32_t*)(a.ws + L.perm);
  uint4* items = (uint4*)(a.ws + L.items);
  uint64_t* bounds = (uint64_t*)(a.ws + L.bounds);
  for (int32_t i = t; i < a.n_tokens; i += kFThreads) perm[i] = s_perm[i];
  for (uint32_t q = (uint32_t)t; q < n_items; q += kFThreads) items[q] = s_items[q];
  const uint64_t wall = (uint64_t)wtot * (uint64_t)a.rows + (uint64_t)n_items * a.item_cost;
  for (int32_t g = t; g <= a.grid; g += kFThreads)
    bounds[g] = weighted_boundary(s_items, n_items, wtot, a.rows, a.item_cost,
                                  wall * (uint64_t)g / (uint64_t)a.grid);
}

// ------------------------------------------------------------ host entries
struct DevInfo {
  int cus = 0;
  int max_lds = 0;        // LDS per workgroup
  // static LDS of the fused-kernel instances, per image kind: the largest over
  // the instances one call may launch (3-slot or 4-slot image)
  int static_lds[2] = {};
  int stack_static_lds = 0;
  bool attr_set = false;
  void* scratch = nullptr;   // device address of this device's copy of `scratch`
};
static std::mutex g_mu;
static DevInfo g_dev[64];

// Workspace of the allocation-free entry point: one copy per device, held
// until the process ends.  In host code `scratch` names a host-side stand-in;
// kernels get the device address that hipGetSymbolAddress returns for the
// current device (DevInfo::scratch), never the array's name.
constexpr size_t kScratchBytes = 256u << 10;
static __device__ __align__(256) uint32_t scratch[kScratchBytes / 4];

static const void* fused_instance(int mode) {
  switch (mode) {
    case 1: return (const void*)fused_kernel<1>;
    case 2: return (const void*)fused_kernel<2>;
    case 3: return (const void*)fused_kernel<3>;
    case 4: return (const void*)fused_kernel<4>;
    case 5: return (const void*)fused_kernel<5>;
    case 6: return (const void*)fused_kernel<6>;
    case 7: return (const void*)fused_kernel<7>;
    case 8: return (const void*)fused_kernel<8>;
    default: return (const void*)fused_kernel<0>;
  }
}

static int dev_info(DevInfo** out, bool want_scratch = false) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SBM_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(SBM_EHIP, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_mu);
  DevInfo& di = g_dev[dev];
  if (!di.cus) {
    int v = 0;
    if ((e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
      return fail(SBM_EHIP, "hipDeviceGetAttribute: %s", hipGetErrorString(e));
    di.cus = v;
    if ((e = hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev)) != hipSuccess)
      return fail(SBM_EHIP, "hipDeviceGetAttribute: %s", hipGetErrorString(e));
    di.max_lds = v;
  }
  if (!di.attr_set) {
    di.static_lds[0] = di.static_lds[1] = 0;
    for (int m = 0; m < kModes; ++m) {
      hipFuncAttributes fa;
      if ((e = hipFuncGetAttributes(&fa, fused_instance(m))) != hipSuccess)
        return fail(SBM_EHIP, "hipFuncGetAttributes: %s", hipGetErrorString(e));
      int& st = di.static_lds[mode_slots(m) == 4 ? 1 : 0];
      st = std::max(st, (int)fa.sharedSizeBytes);
    }
    for (int m = 0; m < kModes; ++m) {
      e = hipFuncSetAttribute(fused_instance(m), hipFuncAttributeMaxDynamicSharedMemorySize,
                              di.max_lds - di.static_lds[mode_slots(m) == 4 ? 1 : 0]);
      if (e != hipSuccess) return fail(SBM_EHIP, "hipFuncSetAttribute: %s", hipGetErrorString(e));
    }
    {
      hipFuncAttributes fa;
      if ((e = hipFuncGetAttributes(&fa, (const void*)stack_kernel<0>)) != hipSuccess)
        return fail(SBM_EHIP, "hipFuncGetAttributes: %s", hipGetErrorString(e));
      di.stack_static_lds = (int)fa.sharedSizeBytes;
      e = hipFuncSetAttribute((const void*)stack_kernel<0>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              di.max_lds - di.stack_static_lds);
      if (e != hipSuccess) return fail(SBM_EHIP, "hipFuncSetAttribute: %s", hipGetErrorString(e));
    }
    di.attr_set = true;
  }
  if (want_scratch && !di.scratch) {
    void* ptr = nullptr;
    if ((e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch))) != hipSuccess || !ptr)
      return fail(SBM_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    di.scratch = ptr;
  }
  *out = &di;
  return SBM_OK;
}

// LDS plan for a shape: tokens per item and rows per chunk.
struct Plan {
  int tcmax, rmax, xcols;
  uint32_t lds_racc, lds_x, lds_total;
};
static bool make_plan(int cols, int max_lds, int static_lds, Plan* p, bool det = false) {
  p->xcols = (cols + (cols >= kSmallCols ? kXWrap : kXPad) + 7) / 8 * 8;
  const int ab = det ? 8 : 4;    // bytes per row accumulator
  // prefer more tokens per item, then the longest row chunks that fit
  for (int tc : {4, 2, 1}) {
    const uint32_t xbytes = (uint32_t)(p->xcols * 6 * tc);
    const int64_t room = (int64_t)max_lds - static_lds - xbytes - 32;
    int64_t rmax = room / (ab * tc) - 2;
    if (rmax > kMaxRmax) rmax = kMaxRmax;
    if (rmax < (tc > 1 ? 256 : 64)) continue;
    p->tcmax = tc;
    p->rmax = (int)rmax;
    p->lds_racc = 0;
    p->lds_x = ((uint32_t)(tc * (rmax + 2) * ab) + 15u) & ~15u;
    p->lds_total = (p->lds_x + xbytes + 15u) & ~15u;
    return true;
  }
  return false;
}

}  // namespace sbm

using namespace sbm;

extern "C" {

int sbm_decode_ref(const uint16_t* codes, const uint32_t* row_off, int32_t rows, int32_t cols,
                   const uint32_t* words, uint8_t* out_sym, uint32_t* bad_rows, void* stream) {
  if (rows < 0 || cols <= 0) return fail(SBM_EINVAL, "bad shape %d x %d", rows, cols);
  if (cols & 1) return fail(SBM_EODD_WIDTH, "cols=%d is odd", cols);
  if (rows == 0) return SBM_OK;
  if (!codes || !row_off || !words || !out_sym) return fail(SBM_EINVAL, "null pointer");
  const int threads = 256;
  const int blocks = (rows + threads - 1) / threads;
  hipLaunchKernelGGL(decode_ref_kernel, dim3(blocks), dim3(threads), 0, (hipStream_t)stream, codes,
                     row_off, rows, cols, words, out_sym, bad_rows);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SBM_EHIP, "decode_ref launch: %s", hipGetErrorString(e));
  return SBM_OK;
}

size_t sbm_workspace_bytes(int32_t n_experts, int32_t n_tokens) {
  if (n_experts < 0 || n_tokens < 0) return 0;
  return (size_t)ws_layout(n_experts, n_tokens).total_words * 4u;
}

}  // extern "C"

// Kernel arguments of one projection call (the kernels read the dictionary
// tag from the image; MFMA tiles and layer fields are set by the callers).
static void fill_args(FusedArgs& a, const uint16_t* codes, const uint32_t* row_off, const uint32_t* bstart,
                      const uint16_t* scales, const sbm_matrix_desc* experts, int32_t n_experts, int32_t rows,
                      int32_t cols, const void* dict_image, const uint16_t* x, const int32_t* expert_ids,
                      int32_t n_tokens, void* y, uint32_t flags, void* workspace, const Plan& plan, int32_t grid) {
  const bool minmax = (flags & SBM_F_MINMAX) != 0;
  a = FusedArgs{};
  a.codes = codes;
  a.row_off = row_off;
  a.bstart = bstart;
  a.scales = scales;
  a.experts = experts;
  a.image = (const DictImage*)dict_image;
  a.x = x;
  a.ids = expert_ids;
  a.y = y;
  a.ws = (uint32_t*)workspace;
  a.rows = rows;
  a.cols = cols;
  a.n_experts = n_experts;
  a.n_tokens = n_tokens;
  a.flags = flags;
  a.colsB = 6u * (uint32_t)cols;
  div_magic(a.colsB, &a.magic_m, &a.magic_s);
  a.rmax = plan.rmax;
  a.tcmax = plan.tcmax;
  a.minmax = minmax ? 1 : 0;
  a.titem = minmax ? plan.tcmax / 2 : plan.tcmax;
  a.xcols = plan.xcols;
  a.lds_racc = plan.lds_racc;
  a.lds_x = plan.lds_x;
  a.grid = grid;
  // an item change costs about as much as kItemChangeBlocks blocks of one-token
  // rows (activation restaging, drain, epilogue); a one-token row of cols
  // columns is about cols / 22 codewords and weighs 4
  a.item_cost = (uint32_t)std::min<int64_t>((int64_t)kRowWeight1 * kItemChangeBlocks * 22 * SBM_BLOCK / cols, 1 << 20);
  a.mfma_rows = 0;
  a.err_out = nullptr;
  a.group_in_lds = n_tokens <= kGroupInLds && n_experts < (1 << 24);
}

// The grouping kernel for calls of more than kGroupInLds tokens.
static int launch_group(const FusedArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(group_kernel, dim3(1), dim3(kThreads), 0, s, a.ids, a.n_tokens, a.n_experts, a.titem, a.rows,
                     a.cols, a.grid, a.item_cost, (int32_t)(a.mfma_rows > 0), a.minmax, a.experts, a.image, a.ws);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SBM_EHIP, "group launch: %s", hipGetErrorString(e));
  return SBM_OK;
}

// The fused call on a given workspace (the caller's, or this device's static
// scratch); err_out, if set, receives a copy of the error word.
static int fused_call(const uint16_t* codes, const uint32_t* row_off, const uint32_t* bstart,
                      const uint16_t* scales, const sbm_matrix_desc* experts, int32_t n_experts, int32_t rows,
                      int32_t cols, const void* dict_image, const uint16_t* x, const int32_t* expert_ids,
                      int32_t n_tokens, void* y, uint32_t flags, void* workspace, size_t workspace_bytes,
                      uint32_t* err_out, bool use_scratch, void* stream) {
  if (n_tokens < 0 || n_tokens > (int32_t)kErrCountMask || n_experts <= 0 || n_experts > (1 << 24))
    return fail(SBM_EINVAL, "bad n_tokens=%d or n_experts=%d", n_tokens, n_experts);
  if (rows <= 0 || rows > (1 << 24) || cols <= 0) return fail(SBM_EINVAL, "bad shape %d x %d", rows, cols);
  if (cols & 1) return fail(SBM_EODD_WIDTH, "cols=%d is odd", cols);
  if ((uint64_t)rows * (uint64_t)cols * 6u + (uint64_t)SBM_BLOCK * 28u * 6u >= (1ull << 30))
    return fail(SBM_ERANGE, "rows*cols too large for 30-bit positions");
  if (flags & ~(SBM_F_RELU | SBM_F_OUT_F32 | SBM_F_IN_RMS | SBM_F_MFMA | SBM_F_MINMAX | SBM_F_IMAGE4 |
                SBM_F_DETERMINISTIC | SBM_F_IN_BF16))
    return fail(SBM_EINVAL, "unknown flags 0x%x", flags);
  if ((flags & SBM_F_IN_BF16) && (flags & SBM_F_MFMA))
    return fail(SBM_EINVAL, "SBM_F_IN_BF16 and SBM_F_MFMA cannot be combined");
  if ((flags & SBM_F_DETERMINISTIC) && (flags & SBM_F_MFMA))
    return fail(SBM_EINVAL, "SBM_F_DETERMINISTIC and SBM_F_MFMA cannot be combined");
  if ((flags & SBM_F_MINMAX) && (flags & SBM_F_MFMA))
    return fail(SBM_EINVAL, "SBM_F_MINMAX and SBM_F_MFMA cannot be combined");
  if ((flags & SBM_F_IMAGE4) && (flags & SBM_F_MFMA))
    return fail(SBM_EINVAL, "SBM_F_IMAGE4 and SBM_F_MFMA cannot be combined");
  if (n_tokens == 0) return SBM_OK;
  if (!codes || !row_off || !bstart || !scales || !experts || !dict_image || !x || !expert_ids || !y ||
      (!workspace && !use_scratch))
    return fail(SBM_EINVAL, "null pointer");
  if (workspace_bytes < sbm_workspace_bytes(n_experts, n_tokens))
    return fail(SBM_ENOSPACE, "workspace %zu < %zu bytes", workspace_bytes,
                sbm_workspace_bytes(n_experts, n_tokens));
  DevInfo* di = nullptr;
  int st = dev_info(&di, use_scratch);
  if (st) return st;
  if (use_scratch) workspace = di->scratch;
  const bool minmax = (flags & SBM_F_MINMAX) != 0;
  const bool det = (flags & SBM_F_DETERMINISTIC) != 0;
  int mode = (flags & SBM_F_MFMA) ? 1 : ((flags & SBM_F_IMAGE4) ? (minmax ? 4 : 3) : (minmax ? 2 : 0));
  if (det) mode = mode == 0 ? 5 : (mode == 2 ? 6 : (mode == 3 ? 7 : 8));
  Plan plan;
  if (!make_plan(cols, di->max_lds, di->static_lds[mode_slots(mode) == 4 ? 1 : 0], &plan, det))
    return fail(SBM_ERANGE, "cols=%d: one token row does not fit in %d bytes of LDS", cols, di->max_lds);
  if (minmax && plan.tcmax < 2)
    return fail(SBM_ERANGE, "cols=%d: the min/max grid needs two activation rows per token in LDS", cols);
  if (minmax && ((uintptr_t)scales & 3u))
    return fail(SBM_EINVAL, "SBM_F_MINMAX: scales must be 4-byte aligned");
  FusedArgs a;
  const int64_t max_items = (int64_t)std::min(n_experts, n_tokens) + n_tokens / (minmax ? plan.tcmax / 2 : plan.tcmax) + 1;
  const int64_t n_upper = max_items * rows;
  int64_t grid = (n_upper + kRowsPerGroup - 1) / kRowsPerGroup;
  if (grid > di->cus) grid = di->cus;
  if (grid > kMaxGrid) grid = kMaxGrid;
  if (grid < 1) grid = 1;
  fill_args(a, codes, row_off, bstart, scales, experts, n_experts, rows, cols, dict_image, x, expert_ids, n_tokens,
            y, flags, workspace, plan, (int32_t)grid);
  a.err_out = err_out;
  if (det) {
    // Every partial sum added to a row accumulator is below 2^28 (a block of
    // 1024 codewords, at most 4 nonzeros each, |x| <= 65504 < 2^16), and a row
    // accumulator receives at most 3 of them per block that touches its row,
    // at most cols / SBM_BLOCK + 2 blocks; 2^62 bounds the integer sums.
    const double terms = 3.0 * ((double)cols / SBM_BLOCK + 2.0);
    a.det_shift = 62 - 28 - (int)std::ceil(std::log2(terms));
  }
  hipStream_t s = (hipStream_t)stream;
  // the in-kernel grouping keeps its sort keys at the start of dynamic LDS
  const uint32_t lds = std::max<uint32_t>(plan.lds_total, kGroupScratch);
  // dense MFMA tiles for heavy experts reuse the same dynamic LDS
  for (int R : {64, 32, 16})
    if ((flags & SBM_F_MFMA) && mfma_lds(R, cols).total <= lds) {
      a.mfma_rows = R;
      break;
    }
  hipError_t e;
  if (!a.group_in_lds && (st = launch_group(a, s))) return st;
  if (a.mfma_rows > 0) hipLaunchKernelGGL(fused_kernel<1>, dim3((unsigned)grid), dim3(kFThreads), lds, s, a);
  else if (mode == 5) hipLaunchKernelGGL(fused_kernel<5>, dim3((unsigned)grid), dim3(kFThreads), lds, s, a);
  else if (mode == 6) hipLaunchKernelGGL(fused_kernel<6>, dim3((unsigned)grid), dim3(kFThreads), lds, s, a);
  else if (mode == 7) hipLaunchKernelGGL(fused_kernel<7>, dim3((unsigned)grid), dim3(kFThreads), lds, s, a);
  else if (mode == 8) hipLaunchKernelGGL(fused_kernel<8>, dim3((unsigned)grid), dim3(kFThreads), lds, s, a);
  else if (mode == 3) hipLaunchKernelGGL(fused_kernel<3>, dim3((unsigned)grid), dim3(kFThreads), lds, s, a);
  else if (mode == 4) hipLaunchKernelGGL(fused_kernel<4>, dim3((unsigned)grid), dim3(kFThreads), lds, s, a);
  else if (a.minmax) hipLaunchKernelGGL(fused_kernel<2>, dim3((unsigned)grid), dim3(kFThreads), lds, s, a);
  else hipLaunchKernelGGL(fused_kernel<0>, dim3((unsigned)grid), dim3(kFThreads), lds, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return fail(SBM_EHIP, "fused launch: %s", hipGetErrorString(e));
  return SBM_OK;
}

extern "C" {

int sbm_moe_fused_decode_matvec(const uint16_t* codes, const uint32_t* row_off,
                                const uint32_t* bstart, const uint16_t* scales,
                                const sbm_matrix_desc* experts, int32_t n_experts, int32_t rows,
                                int32_t cols, const void* dict_image, const uint16_t* x,
                                const int32_t* expert_ids, int32_t n_tokens, void* y,
                                uint32_t flags, void* workspace, size_t workspace_bytes,
                                void* stream) {
  return fused_call(codes, row_off, bstart, scales, experts, n_experts, rows, cols, dict_image, x, expert_ids,
                    n_tokens, y, flags, workspace, workspace_bytes, nullptr, false, stream);
}

int sbm_moe_fused_decode_matvec_noalloc(const uint16_t* codes, const uint32_t* row_off,
                                        const uint32_t* bstart, const uint16_t* scales,
                                        const sbm_matrix_desc* experts, int32_t n_experts, int32_t rows,
                                        int32_t cols, const void* dict_image, const uint16_t* x,
                                        const int32_t* expert_ids, int32_t n_tokens, void* y,
                                        uint32_t flags, uint32_t* error_word, void* stream) {
  if (n_tokens > 0 && n_experts > 0 && sbm_workspace_bytes(n_experts, n_tokens) > kScratchBytes)
    return fail(SBM_ERANGE, "%d experts x %d tokens need %zu bytes of workspace; the allocation-free call "
                "holds %zu (use sbm_moe_fused_decode_matvec with a workspace)", n_experts, n_tokens,
                sbm_workspace_bytes(n_experts, n_tokens), kScratchBytes);
  return fused_call(codes, row_off, bstart, scales, experts, n_experts, rows, cols, dict_image, x, expert_ids,
                    n_tokens, y, flags, nullptr, kScratchBytes, error_word, true, stream);
}

static size_t align16(size_t b) { return (b + 15u) & ~(size_t)15u; }

size_t sbm_layers_workspace_bytes(int32_t n_layers, int32_t n_experts, int32_t n_tokens) {
  if (n_layers <= 0 || n_experts < 0 || n_tokens < 0) return 0;
  const size_t phases = 2u * (size_t)n_layers;
  return align16(((size_t)kSyncHdr + phases * (size_t)n_tokens) * 4u) +
         phases * align16(sbm_workspace_bytes(n_experts, n_tokens));
}

size_t sbm_ffn_workspace_bytes(int32_t n_experts, int32_t n_tokens) {
  return sbm_layers_workspace_bytes(1, n_experts, n_tokens);
}

}  // extern "C"

// n_layers layers of (up, ReLU, down) in one launch: the layer call is n_layers = 1.
static int layers_call(const sbm_projection* up, const sbm_projection* down, int32_t n_layers,
                       const void* dict_image, const uint16_t* x, const int32_t* expert_ids, int32_t n_tokens,
                       uint16_t* h, void* y, uint32_t flags, void* workspace, size_t workspace_bytes, void* stream) {
  if (!up || !down) return fail(SBM_EINVAL, "null projection");
  if (n_layers <= 0 || n_layers > kMaxLayers)
    return fail(SBM_EINVAL, "n_layers=%d outside 1..%d (longer stacks: one call per %d layers)", n_layers,
                kMaxLayers, kMaxLayers);
  if (n_tokens < 0 || n_tokens > (int32_t)kErrCountMask) return fail(SBM_EINVAL, "bad n_tokens=%d", n_tokens);
  for (int32_t l = 0; l < n_layers; ++l) {
    const sbm_projection* u = up + l;
    const sbm_projection* d = down + l;
    if (u->n_experts <= 0 || u->n_experts > (1 << 24) || u->n_experts != d->n_experts ||
        u->n_experts != up->n_experts)
      return fail(SBM_EINVAL, "layer %d: the projections must hold the same experts as layer 0 (%d, %d, %d)", l,
                  u->n_experts, d->n_experts, up->n_experts);
    for (const sbm_projection* q : {u, d}) {
      if (q->rows <= 0 || q->rows > (1 << 24) || q->cols <= 0)
        return fail(SBM_EINVAL, "bad shape %d x %d", q->rows, q->cols);
      if (q->cols & 1) return fail(SBM_EODD_WIDTH, "cols=%d is odd", q->cols);
      if (q->cols < kSmallCols)
        return fail(SBM_EINVAL, "cols=%d: the layer call needs rows of at least %d columns (use two "
                    "sbm_moe_fused_decode_matvec calls)", q->cols, kSmallCols);
      if ((uint64_t)q->rows * (uint64_t)q->cols * 6u + (uint64_t)SBM_BLOCK * 28u * 6u >= (1ull << 30))
        return fail(SBM_ERANGE, "rows*cols too large for 30-bit positions");
      if (!q->codes || !q->row_off || !q->bstart || !q->scales || !q->experts)
        return fail(SBM_EINVAL, "null pointer");
    }
    if (u->rows != up->rows || u->cols != up->cols || d->rows != down->rows || d->cols != down->cols)
      return fail(SBM_EINVAL, "layer %d: every layer must have layer 0's shapes", l);
  }
  if (up->rows != down->cols)
    return fail(SBM_EINVAL, "up rows (%d) must equal down cols (%d): h is their common width", up->rows, down->cols);
  if (n_layers > 1 && down->rows != up->cols)
    return fail(SBM_EINVAL, "down rows (%d) must equal up cols (%d): each layer's output feeds the next",
                down->rows, up->cols);
  if (flags & ~(SBM_F_OUT_F32 | SBM_F_IN_RMS | SBM_F_IN_BF16))
    return fail(SBM_EINVAL, "unknown or unsupported flags 0x%x", flags);
  if (n_layers > 1 && (flags & SBM_F_OUT_F32))
    return fail(SBM_EINVAL, "SBM_F_OUT_F32: one layer only (every layer's fp16 output feeds the next)");
  if ((uint64_t)n_tokens * (uint64_t)std::max(down->cols, up->cols) * 2u >= (1ull << 31))
    return fail(SBM_ERANGE, "activations too large");
  if (n_tokens == 0) return SBM_OK;
  if (!dict_image || !x || !expert_ids || !h || !y || !workspace) return fail(SBM_EINVAL, "null pointer");
  if ((uintptr_t)workspace & 15u) return fail(SBM_EINVAL, "workspace must be 16-byte aligned");
  const size_t need = sbm_layers_workspace_bytes(n_layers, up->n_experts, n_tokens);
  if (workspace_bytes < need) return fail(SBM_ENOSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
  DevInfo* di = nullptr;
  int st = dev_info(&di);
  if (st) return st;
  Plan pu, pd;
  if (!make_plan(up->cols, di->max_lds, di->stack_static_lds, &pu) ||
      !make_plan(down->cols, di->max_lds, di->stack_static_lds, &pd))
    return fail(SBM_ERANGE, "a token row does not fit in %d bytes of LDS", di->max_lds);
  // Each phase is cut into as many slices as its rows fill at kRowsPerGroup
  // rows per workgroup (as a projection call is), at most one per CU; the
  // launch holds the larger count, and workgroups past a phase's count skip it.
  auto phase_grid = [&](const sbm_projection* p, const Plan& pl) {
    const int64_t max_items = (int64_t)std::min(p->n_experts, n_tokens) + n_tokens / pl.tcmax + 1;
    const int64_t g = (max_items * p->rows + kRowsPerGroup - 1) / kRowsPerGroup;
    return (int32_t)std::max<int64_t>(1, std::min<int64_t>(g, std::min(di->cus, kMaxGrid)));
  };
  const int32_t grid_u = phase_grid(up, pu), grid_d = phase_grid(down, pd), grid = std::max(grid_u, grid_d);
  uint32_t* sync = (uint32_t*)workspace;
  const size_t phase_bytes = align16(sbm_workspace_bytes(up->n_experts, n_tokens));
  unsigned char* ws0 = (unsigned char*)workspace + align16(((size_t)kSyncHdr + 2u * (size_t)n_layers *
                                                                                   (size_t)n_tokens) * 4u);
  FusedArgs ua, da;
  fill_args(ua, up->codes, up->row_off, up->bstart, up->scales, up->experts, up->n_experts, up->rows, up->cols,
            dict_image, x, expert_ids, n_tokens, h, SBM_F_RELU | (flags & (SBM_F_IN_RMS | SBM_F_IN_BF16)), ws0, pu,
            grid_u);
  fill_args(da, down->codes, down->row_off, down->bstart, down->scales, down->experts, down->n_experts, down->rows,
            down->cols, dict_image, h, expert_ids, n_tokens, y, flags & SBM_F_OUT_F32, ws0 + phase_bytes, pd, grid_d);
  ua.sync_err = da.sync_err = sync + 1;
  // a layer call's phases weigh an item change a little more (its staging
  // waits for other workgroups' rows)
  ua.item_cost = ua.item_cost * kLayerItemChangeBlocks / kItemChangeBlocks;
  da.item_cost = da.item_cost * kLayerItemChangeBlocks / kItemChangeBlocks;
  da.x_bytes = (uint32_t)((uint64_t)n_tokens * (uint64_t)down->cols * 2u);
  LayerTab tab;
  memset(&tab, 0, sizeof(tab));
  for (int32_t l = 0; l < n_layers; ++l) {
    tab.up[l] = LayerProj{up[l].codes, up[l].row_off, up[l].bstart, up[l].scales, up[l].experts};
    tab.dn[l] = LayerProj{down[l].codes, down[l].row_off, down[l].bstart, down[l].scales, down[l].experts};
  }
  tab.h = h;
  tab.y = (uint16_t*)y;
  tab.ws_words = (uint32_t)(phase_bytes / 4u);
  tab.n_layers = n_layers;
  hipStream_t s = (hipStream_t)stream;
  if (ua.group_in_lds && n_layers > 1) {
    // every phase grouped ahead by one launch (the layer launch then groups
    // nothing; with one layer, grouping inside the layer launch is faster)
    hipLaunchKernelGGL(stack_plan_kernel, dim3((unsigned)(2 * n_layers)), dim3(kFThreads), kGroupScratch, s, ua, da,
                       tab, sync);
    const hipError_t pe = hipGetLastError();
    if (pe != hipSuccess) return fail(SBM_EHIP, "grouping launch: %s", hipGetErrorString(pe));
    ua.group_in_lds = da.group_in_lds = 0;
  } else if (!ua.group_in_lds) {
    // more tokens than the in-kernel grouping takes: every phase grouped by
    // one launch, each into its phase's part of the workspace
    hipLaunchKernelGGL(stack_group_kernel, dim3((unsigned)(2 * n_layers)), dim3(kThreads), 0, s, ua, da, tab, sync);
    const hipError_t ge = hipGetLastError();
    if (ge != hipSuccess) return fail(SBM_EHIP, "grouping launch: %s", hipGetErrorString(ge));
  }
  const uint32_t lds = std::max<uint32_t>(std::max(pu.lds_total, pd.lds_total), kGroupScratch);
  hipLaunchKernelGGL(stack_kernel<0>, dim3((unsigned)grid), dim3(kFThreads), lds, s, ua, da, tab, sync);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SBM_EHIP, "layer launch: %s", hipGetErrorString(e));
  return SBM_OK;
}

extern "C" {

int sbm_moe_fused_ffn(const sbm_projection* up, const sbm_projection* down, const void* dict_image,
                      const uint16_t* x, const int32_t* expert_ids, int32_t n_tokens, uint16_t* h, void* y,
                      uint32_t flags, void* workspace, size_t workspace_bytes, void* stream) {
  return layers_call(up, down, 1, dict_image, x, expert_ids, n_tokens, h, y, flags, workspace, workspace_bytes,
                     stream);
}

int sbm_moe_fused_layers(const sbm_projection* up, const sbm_projection* down, int32_t n_layers,
                         const void* dict_image, const uint16_t* x, const int32_t* expert_ids, int32_t n_tokens,
                         uint16_t* h, uint16_t* y, uint32_t flags, void* workspace, size_t workspace_bytes,
                         void* stream) {
  return layers_call(up, down, n_layers, dict_image, x, expert_ids, n_tokens, h, y, flags, workspace,
                     workspace_bytes, stream);
}

int sbm_workspace_error(const void* workspace, uint32_t* out_error, void* stream) {
  if (!workspace || !out_error) return fail(SBM_EINVAL, "null pointer");
  hipError_t e = hipMemcpyAsync(out_error, workspace, 4, hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return fail(SBM_EHIP, "reading the error word: %s", hipGetErrorString(e));
  return SBM_OK;
}

}  // extern "C"
