// GPU generation and encoding of counter-based synthetic expert stacks.
//
// The QMoE page ("QMoE: Practical Sub-1-Bit Compression of Trillion-Parameter
// Models", Executive Summary and section "Natural sparsity") describes a
// 1.6T-parameter c2048 stack held in under 160 GB at ~0.8 bit per parameter,
// with about 88.6% zeros.  Such a stack cannot be materialised as ternary
// symbols anywhere, so it is generated here row by row from a counter-based
// generator and encoded on the fly with the same greedy trie walk as the host
// encoder ("Encoding": trie over the dictionary, longest prefix, rows
// independent).
//
// Generator (shared definition with the seeded-input module on the host):
//   SplitMix64 output number i for state s is mix64(s + i*0x9E3779B97F4A7C15)
//   (Steele, Lea, Flood 2014; Vigna's reference code).
//   Matrix key      = output (m+1) for state `seed`, m = (layer*E + e)*2 + mat.
//   Symbols of row r, column j: 16-bit lane j%4 of output r*ceil(cols/4)+j/4+1
//     for the matrix key; v < Z -> 0, odd v -> 2 (positive), even v -> 1.
//   Scale index of row r: top 12 bits of output 2^40 + r + 1.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "sbm_internal.h"

namespace sbm {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
constexpr int32_t kRoot = SBM_DICT_ENTRIES;

__host__ __device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__host__ __device__ __forceinline__ uint64_t splitmix_at(uint64_t state, uint64_t i) {
  return mix64(state + i * kGamma);
}

struct GenArgs {
  uint64_t seed;
  int32_t layer, n_experts, mat, rows, cols;
  uint32_t zth;                 // zero threshold on 16-bit draws
  const int32_t* trie;          // child[(65536+1)*9]
  uint32_t* row_counts;         // count pass: [E*rows]
  const uint32_t* row_off;      // write pass: [E*(rows+1)]
  const sbm_matrix_desc* desc;  // write pass
  uint16_t* codes;
  uint32_t* bstart;
  const uint16_t* scale_table;  // 4096 fp16
  uint16_t* scales;             // [E*rows]
};

// One thread per row: generate the row's symbols pair by pair and walk the
// trie; the count pass counts codewords, the write pass stores them, the
// block starts that fall in the row, and the row scale.
template <bool WRITE>
__global__ __launch_bounds__(256) void gen_walk(GenArgs g) {
  const int64_t gr = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // global row
  if (gr >= (int64_t)g.n_experts * g.rows) return;
  const int32_t e = (int32_t)(gr / g.rows), r = (int32_t)(gr - (int64_t)e * g.rows);
  const uint64_t m = ((uint64_t)g.layer * g.n_experts + e) * 2 + g.mat;
  const uint64_t key = splitmix_at(g.seed, m + 1);
  const uint64_t w = (uint64_t)(g.cols + 3) / 4;
  uint32_t n = 0;
  uint64_t out_base = 0;
  uint32_t off0 = 0;
  uint64_t blk_base = 0;
  if (WRITE) {
    const sbm_matrix_desc d = g.desc[e];
    off0 = g.row_off[(int64_t)e * (g.rows + 1) + r];
    out_base = d.code_base;
    blk_base = d.blk_base;
    const uint64_t hs = splitmix_at(key, (1ull << 40) + (uint64_t)r + 1);
    g.scales[d.scale_base + r] = g.scale_table[hs >> 52];
  }
  int32_t cur = kRoot;
  int32_t start = 0;    // column where the current codeword starts
  for (int32_t j = 0; j < g.cols; j += 4) {
    const uint64_t h = splitmix_at(key, (uint64_t)r * w + (uint64_t)(j / 4) + 1);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int32_t col = j + 2 * q;
      if (col >= g.cols) break;
      const uint32_t v0 = (uint32_t)(h >> (32 * q)) & 0xFFFFu;
      const uint32_t v1 = (uint32_t)(h >> (32 * q + 16)) & 0xFFFFu;
      const uint32_t s0 = v0 < g.zth ? 0u : ((v0 & 1u) ? 2u : 1u);
      const uint32_t s1 = v1 < g.zth ? 0u : ((v1 & 1u) ? 2u : 1u);
      const int32_t pr = (int32_t)(3 * s0 + s1);
      const int32_t nx = g.trie[(int64_t)cur * 9 + pr];
      if (nx >= 0) {
        cur = nx;
      } else {
        if (WRITE) {
          const uint32_t idx = off0 + n;
          g.codes[out_base + idx] = (uint16_t)cur;
          if ((idx % SBM_BLOCK) == 0) g.bstart[blk_base + idx / SBM_BLOCK] = (uint32_t)r * g.cols + start;
        }
        ++n;
        cur = g.trie[(int64_t)kRoot * 9 + pr];
        start = col;
      }
    }
  }
  if (cur != kRoot) {
    if (WRITE) {
      const uint32_t idx = off0 + n;
      g.codes[out_base + idx] = (uint16_t)cur;
      if ((idx % SBM_BLOCK) == 0) g.bstart[blk_base + idx / SBM_BLOCK] = (uint32_t)r * g.cols + start;
    }
    ++n;
  }
  if (!WRITE) g.row_counts[gr] = n;
}

// Exclusive scan of one matrix's row counts into its rows+1 row offsets
// (one workgroup per matrix).
__global__ __launch_bounds__(1024) void gen_row_scan(const uint32_t* __restrict__ counts, int32_t rows,
                                                     uint32_t* __restrict__ row_off) {
  __shared__ uint32_t part[1024];
  const int32_t e = blockIdx.x;
  const uint32_t* c = counts + (int64_t)e * rows;
  uint32_t* o = row_off + (int64_t)e * (rows + 1);
  const int32_t per = (rows + 1023) / 1024;
  const int32_t r0 = threadIdx.x * per;
  uint32_t s = 0;
  for (int32_t i = 0; i < per && r0 + i < rows; ++i) s += c[r0 + i];
  part[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t run = 0;
    for (int i = 0; i < 1024; ++i) {
      const uint32_t t = part[i];
      part[i] = run;
      run += t;
    }
    o[rows] = run;
  }
  __syncthreads();
  uint32_t run = part[threadIdx.x];
  for (int32_t i = 0; i < per && r0 + i < rows; ++i) {
    o[r0 + i] = run;
    run += c[r0 + i];
  }
}

// Matrix descriptors: codeword bases (multiples of SBM_CODE_ALIGN), block
// bases and the total, from the per-matrix codeword counts (one workgroup).
__global__ __launch_bounds__(1024) void gen_desc(const uint32_t* __restrict__ row_off, int32_t E, int32_t rows,
                                                 int32_t cols, uint32_t dict_tag, sbm_matrix_desc* __restrict__ desc,
                                                 uint64_t* __restrict__ totals) {
  __shared__ uint64_t pc[1024], pb[1024];
  const int32_t per = (E + 1023) / 1024;
  const int32_t e0 = threadIdx.x * per;
  uint64_t sc = 0, sb = 0;
  for (int32_t i = 0; i < per && e0 + i < E; ++i) {
    const uint64_t n = row_off[(int64_t)(e0 + i) * (rows + 1) + rows];
    sc += (n + SBM_CODE_ALIGN - 1) / SBM_CODE_ALIGN * SBM_CODE_ALIGN;
    sb += (n + SBM_BLOCK - 1) / SBM_BLOCK;
  }
  pc[threadIdx.x] = sc;
  pb[threadIdx.x] = sb;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t rc = 0, rb = 0;
    for (int i = 0; i < 1024; ++i) {
      const uint64_t a = pc[i], b = pb[i];
      pc[i] = rc;
      pb[i] = rb;
      rc += a;
      rb += b;
    }
    totals[0] = rc;
    totals[1] = rb;
  }
  __syncthreads();
  uint64_t rc = pc[threadIdx.x], rb = pb[threadIdx.x];
  for (int32_t i = 0; i < per && e0 + i < E; ++i) {
    const int32_t e = e0 + i;
    const uint64_t n = row_off[(int64_t)e * (rows + 1) + rows];
    sbm_matrix_desc d;
    d.code_base = rc;
    d.off_base = (uint64_t)e * (rows + 1);
    d.scale_base = (uint64_t)e * rows;
    d.blk_base = rb;
    d.n_codes = (uint32_t)n;
    d.rows = rows;
    d.cols = cols;
    d.dict_tag = dict_tag;
    desc[e] = d;
    rc += (n + SBM_CODE_ALIGN - 1) / SBM_CODE_ALIGN * SBM_CODE_ALIGN;
    rb += (n + SBM_BLOCK - 1) / SBM_BLOCK;
  }
}

static int check_gen(int32_t layer, int32_t E, int32_t mat, int32_t rows, int32_t cols) {
  if (layer < 0 || E <= 0 || (mat != 0 && mat != 1) || rows <= 0 || cols <= 0)
    return fail(SBM_EINVAL, "bad generator arguments");
  if (cols & 1) return fail(SBM_EODD_WIDTH, "cols=%d is odd", cols);
  if ((uint64_t)rows * cols >= (1ull << 32)) return fail(SBM_ERANGE, "matrix too large");
  if ((uint64_t)E * rows >= (1ull << 31)) return fail(SBM_ERANGE, "too many rows");
  return SBM_OK;
}

}  // namespace sbm

using namespace sbm;

extern "C" {

int sbm_gen_count(uint64_t seed, int32_t layer, int32_t n_experts, int32_t mat, int32_t rows, int32_t cols,
                  uint32_t zero_threshold16, const int32_t* trie, uint32_t* row_counts, void* stream) {
  int st = check_gen(layer, n_experts, mat, rows, cols);
  if (st) return st;
  if (!trie || !row_counts) return fail(SBM_EINVAL, "null pointer");
  GenArgs g = {};
  g.seed = seed;
  g.layer = layer;
  g.n_experts = n_experts;
  g.mat = mat;
  g.rows = rows;
  g.cols = cols;
  g.zth = zero_threshold16;
  g.trie = trie;
  g.row_counts = row_counts;
  const int64_t total = (int64_t)n_experts * rows;
  hipLaunchKernelGGL(gen_walk<false>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, (hipStream_t)stream, g);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SBM_EHIP, "gen_count launch: %s", hipGetErrorString(e));
  return SBM_OK;
}

int sbm_gen_layout(const uint32_t* row_counts, int32_t n_experts, int32_t rows, int32_t cols, uint32_t* row_off,
                   sbm_matrix_desc* desc, uint64_t* totals, uint64_t dict_checksum, void* stream) {
  if (!row_counts || !row_off || !desc || !totals || n_experts <= 0 || rows <= 0 || cols <= 0)
    return fail(SBM_EINVAL, "bad layout arguments");
  hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL(gen_row_scan, dim3(n_experts), dim3(1024), 0, s, row_counts, rows, row_off);
  hipLaunchKernelGGL(gen_desc, dim3(1), dim3(1024), 0, s, row_off, n_experts, rows, cols, (uint32_t)dict_checksum,
                     desc, totals);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SBM_EHIP, "gen_layout launch: %s", hipGetErrorString(e));
  return SBM_OK;
}

int sbm_gen_write(uint64_t seed, int32_t layer, int32_t n_experts, int32_t mat, int32_t rows, int32_t cols,
                  uint32_t zero_threshold16, const int32_t* trie, const uint32_t* row_off,
                  const sbm_matrix_desc* desc, uint16_t* codes, uint32_t* bstart, const uint16_t* scale_table,
                  uint16_t* scales, void* stream) {
  int st = check_gen(layer, n_experts, mat, rows, cols);
  if (st) return st;
  if (!trie || !row_off || !desc || !codes || !bstart || !scale_table || !scales)
    return fail(SBM_EINVAL, "null pointer");
  GenArgs g = {};
  g.seed = seed;
  g.layer = layer;
  g.n_experts = n_experts;
  g.mat = mat;
  g.rows = rows;
  g.cols = cols;
  g.zth = zero_threshold16;
  g.trie = trie;
  g.row_off = row_off;
  g.desc = desc;
  g.codes = codes;
  g.bstart = bstart;
  g.scale_table = scale_table;
  g.scales = scales;
  const int64_t total = (int64_t)n_experts * rows;
  hipLaunchKernelGGL(gen_walk<true>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, (hipStream_t)stream, g);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SBM_EHIP, "gen_write launch: %s", hipGetErrorString(e));
  return SBM_OK;
}

}  // extern "C"

// ------------------------------------------------------------------ stack glue
// Between stacked MoE layers the transformer block the pages' model would run
// is absent; to keep fp16 activations in range the harness normalises each
// token: x_next = y / sqrt(mean(y^2)) (fp32 arithmetic, fp16 result).  This is
// benchmark glue, not part of the method.  One workgroup per token.
namespace sbm {
__global__ __launch_bounds__(256) void rms_glue_kernel(const uint16_t* __restrict__ y, int32_t d,
                                                       uint16_t* __restrict__ out) {
  __shared__ float part[256];
  const _Float16* yr = (const _Float16*)y + (int64_t)blockIdx.x * d;
  _Float16* orow = (_Float16*)out + (int64_t)blockIdx.x * d;
  float s = 0.f;
  for (int32_t i = threadIdx.x; i < d; i += 256) {
    const float v = (float)yr[i];
    s += v * v;
  }
  part[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  const float ms = part[0] / (float)d;
  const float inv = ms > 0.f ? 1.0f / sqrtf(ms) : 1.0f;
  for (int32_t i = threadIdx.x; i < d; i += 256) orow[i] = (_Float16)((float)yr[i] * inv);
}
}  // namespace sbm

extern "C" int sbm_rms_glue(const uint16_t* y, int32_t n_tokens, int32_t d, uint16_t* x_out, void* stream) {
  if (n_tokens < 0 || d <= 0) return sbm::fail(SBM_EINVAL, "bad shape");
  if (n_tokens == 0) return SBM_OK;
  if (!y || !x_out) return sbm::fail(SBM_EINVAL, "null pointer");
  hipLaunchKernelGGL(sbm::rms_glue_kernel, dim3(n_tokens), dim3(256), 0, (hipStream_t)stream, y, d, x_out);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return sbm::fail(SBM_EHIP, "rms_glue launch: %s", hipGetErrorString(e));
  return SBM_OK;
}

// ------------------------------------------------------------ bandwidth probe
// The practical read bandwidth of the device, the denominator the
// cache-amplification page uses for its host roofline ("Results", host
// roofline table: a measured GPU device copy next to the nominal figure):
// a grid-stride stream of 16-byte loads over the buffer, folded into one
// word per workgroup so the loads cannot be dropped.
namespace sbm {
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t* __restrict__ p, uint64_t n16,
                                                          uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const uint64_t stride = (uint64_t)gridDim.x * 256u;
  for (uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x; i < n16; i += 4 * stride) {
    u32x4_t v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = i + k * stride < n16 ? __builtin_nontemporal_load(p + i + k * stride)
                                                           : u32x4_t{0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < 4; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  __shared__ uint32_t s[256];
  s[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int i = 0; i < 256; ++i) r ^= s[i];
    sink[blockIdx.x] = r;
  }
}
}  // namespace sbm

extern "C" int sbm_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, uint32_t sink_words, void* stream) {
  if (!buf || !sink || sink_words == 0) return sbm::fail(SBM_EINVAL, "null pointer or empty sink");
  if (((uintptr_t)buf & 15u) || (bytes & 15u)) return sbm::fail(SBM_EINVAL, "buffer and size must be multiples of 16");
  if (bytes == 0) return SBM_OK;
  const uint64_t n16 = bytes / 16u;
  const unsigned grid = (unsigned)std::min<uint64_t>(sink_words, std::max<uint64_t>(1, n16 / 1024));
  hipLaunchKernelGGL(sbm::stream_read_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const sbm::u32x4_t*)buf, n16,
                     sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return sbm::fail(SBM_EHIP, "stream_read launch: %s", hipGetErrorString(e));
  return SBM_OK;
}
