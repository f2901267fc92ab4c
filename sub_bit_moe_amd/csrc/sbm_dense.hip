// Block-parallel decode of one matrix to dense fp16 ternary values, the first
// step of the two-launch alternative to the fused kernel: decompress, then a
// dense GEMM on the matrix cores ([QMoE] "The GPU Decoding Kernel" names
// decompress-then-multiply as the path its fused kernel avoids; the
// cache-amplification page prices it as dense weights written, read back and
// read again).  Output element (r, j) is -1, 0 or +1 as fp16 (the row scale
// stays out, for the GEMM's epilogue), so the result is exact.
//
// One wave per 1024-codeword block: the block's codewords cover the contiguous
// element range [bstart[b], bstart[b+1]) of the row-major matrix (block starts
// are linear positions row * cols + col).  The wave issues the zero fill of
// that range (16-byte stores on its 16-byte aligned part), loads its 16
// codewords per lane with two 16-byte loads, looks each one up in the compact
// table the fused kernel uses (read from global memory, where it stays in
// L2: one workgroup per block leaves no time to copy 60 KB into LDS first),
// adds the signs from the codeword's low bits, waits for the fill, and writes
// each nonzero.  No division by the row width is needed.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "sbm_internal.h"

namespace sbm {
namespace {

constexpr int kDThreads = 128;    // 2 waves, one block each
constexpr int kDWaves = kDThreads / 64;
constexpr int kDK = SBM_BLOCK / 64;   // codewords per lane
static_assert(kDK == 16, "two 16-byte code loads per lane");
constexpr uint16_t kMinusOne = 0xBC00u, kPlusOne = 0x3C00u;   // fp16 -1.0, +1.0

__device__ __forceinline__ uint32_t wave_excl_scan(uint32_t v, uint32_t lane) {
  uint32_t s = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t t = __shfl_up(s, d, 64);
    if (lane >= (uint32_t)d) s += t;
  }
  return s - v;
}

__global__ __launch_bounds__(kDThreads) void decode_dense_kernel(const uint16_t* __restrict__ codes,
                                                                 uint32_t n_codes,
                                                                 const uint32_t* __restrict__ bstart,
                                                                 uint64_t n_elems, const DictImage* __restrict__ im,
                                                                 uint32_t dict_tag, uint16_t* __restrict__ out,
                                                                 uint32_t* bad, int vec_codes) {
  const uint4 hdr = *(const uint4*)im;       // magic, version, split H, n_tab (the same for every thread)
  const bool ok = hdr.x == kImageMagic && hdr.y == kImageVersion && hdr.z <= SBM_DICT_ENTRIES &&
                  hdr.w == hdr.z + (SBM_DICT_ENTRIES - hdr.z + 7u) / 8u && hdr.w <= kTabEntries;
  if (!ok) {
    if (blockIdx.x == 0 && threadIdx.x == 0) *bad = 1u;
    return;
  }
  if ((uint32_t)im->checksum != dict_tag) {      // codes of another dictionary: decoding would mislabel them
    if (blockIdx.x == 0 && threadIdx.x == 0) *bad = 2u;
    return;
  }
  const uint32_t* tab = im->tab;             // every index below is < n_tab (see table_index in the fused kernel)
  const uint32_t split7 = 7u * hdr.z;
  const uint32_t nblk = (n_codes + SBM_BLOCK - 1) / SBM_BLOCK;
  const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t* out2 = (uint32_t*)out;           // fp16 pairs: block spans start and end at even positions
  for (uint32_t b = blockIdx.x * kDWaves + wave; b < nblk; b += gridDim.x * kDWaves) {
    const uint64_t e1 = b + 1 < nblk ? (uint64_t)bstart[b + 1] : n_elems;
    const uint64_t p1 = std::min<uint64_t>(e1, n_elems);
    const uint64_t p0 = std::min<uint64_t>(bstart[b], p1);
    {
      // [p0, p1) starts and ends at even elements; the part whose addresses
      // are 16-byte aligned is filled with 16-byte stores, the pairs before
      // and after it (at most 3 each) with 4-byte stores.  out is 4-byte
      // aligned, so `off` (its element offset within 16 bytes) is even.
      const uint64_t off = ((uintptr_t)out >> 1) & 7u;
      const uint64_t a8 = std::min<uint64_t>(((p0 + off + 7u) & ~7ull) - off, p1);
      const uint64_t b8 = std::max<uint64_t>(((p1 + off) & ~7ull) - off, a8);
      uint4* out16 = (uint4*)(out - off);        // 16-byte aligned; element e sits in piece (e + off) / 8
      for (uint64_t q = (a8 + off) / 8 + lane; q < (b8 + off) / 8; q += 64) out16[q] = make_uint4(0u, 0u, 0u, 0u);
      const uint64_t h = p0 / 2 + lane;
      if (h < a8 / 2) out2[h] = 0u;
      const uint64_t t = b8 / 2 + lane;
      if (t < p1 / 2) out2[t] = 0u;
    }
    // this lane's codewords: two 16-byte loads when the stream is 16-byte
    // aligned (streams of a stack are), else, and at the stream's end, one at a time
    const uint32_t i0 = b * SBM_BLOCK + lane * kDK;
    uint32_t c[kDK];
    if (vec_codes && i0 + kDK <= n_codes) {
      const uint4 lo = *(const uint4*)(codes + i0), hi = *(const uint4*)(codes + i0 + 8);
      const uint32_t wds[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
      for (int j = 0; j < kDK; ++j) c[j] = (j & 1) ? (wds[j >> 1] >> 16) : (wds[j >> 1] & 0xFFFFu);
    } else {
#pragma unroll
      for (int j = 0; j < kDK; ++j) c[j] = i0 + j < n_codes ? (uint32_t)codes[i0 + j] : 0xFFFFFFFFu;
    }
    uint32_t w[kDK];
#pragma unroll
    for (int j = 0; j < kDK; ++j) {
      const uint32_t e = c[j] + split7;
      w[j] = c[j] == 0xFFFFFFFFu ? 0u : tab[min(c[j], e >> 3)];
    }
    uint32_t tot = 0;                         // 6 * symbols of the lane's codewords
#pragma unroll
    for (int j = 0; j < kDK; ++j) {
      if (c[j] == 0xFFFFFFFFu) {
        w[j] = 0x00040404u;                   // past the stream: no symbols, empty slots
      } else {
        w[j] += ((((c[j] + split7) & 7u) * 0x8102u) & 0x20202u);
      }
      tot += w[j] >> 24;
    }
    const uint32_t before6 = wave_excl_scan(tot, lane);
    uint64_t pos = p0 + ((uint64_t)before6 * 0xAAAAAAABull >> 34);   // before6 / 6, exact
    __builtin_amdgcn_s_waitcnt(0x0F70);      // vmcnt(0): the zeros have landed before the nonzeros
#pragma unroll
    for (int j = 0; j < kDK; ++j) {
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const uint32_t byte = (w[j] >> (8 * i)) & 0xFFu;
        const uint32_t p = (byte * 171u) >> 10;          // byte / 6 for byte < 256
        const uint32_t k = byte - 6u * p;                // 0: -1, 2: +1, 4: empty
        const uint64_t q = pos + p;
        if (k != 4u && q < p1) out[q] = k == 0u ? kMinusOne : kPlusOne;
      }
      pos += (w[j] >> 24) / 6u;
    }
  }
}

}  // namespace
}  // namespace sbm

using namespace sbm;

extern "C" int sbm_decode_dense(const uint16_t* codes, uint64_t n_codes, const uint32_t* bstart, int32_t rows,
                                int32_t cols, const void* dict_image, uint32_t dict_tag, uint16_t* out_fp16,
                                uint32_t* bad, void* stream) {
  if (rows < 0 || cols <= 0) return fail(SBM_EINVAL, "bad shape %d x %d", rows, cols);
  if (cols & 1) return fail(SBM_EODD_WIDTH, "cols=%d is odd", cols);
  if (rows == 0) return SBM_OK;
  const uint64_t n_elems = (uint64_t)rows * (uint64_t)cols;
  if (n_elems > 0xFFFFFFFFull) return fail(SBM_ERANGE, "rows*cols above the 32-bit block start positions");
  if (n_codes == 0 || n_codes > 0xFFFFFFFFull)
    return fail(SBM_EINVAL, "n_codes=%llu for %d rows", (unsigned long long)n_codes, rows);
  if (!codes || !bstart || !dict_image || !out_fp16 || !bad) return fail(SBM_EINVAL, "null pointer");
  if ((uintptr_t)out_fp16 & 3u) return fail(SBM_EINVAL, "out must be 4-byte aligned");
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return fail(SBM_EHIP, "device query: %s", hipGetErrorString(e));
  const uint64_t nblk = (n_codes + SBM_BLOCK - 1) / SBM_BLOCK;
  const uint64_t want = (nblk + kDWaves - 1) / kDWaves;   // one block per wave
  const unsigned grid = (unsigned)std::max<uint64_t>(1, std::min<uint64_t>(want, 64ull * (uint64_t)cus));
  hipLaunchKernelGGL(decode_dense_kernel, dim3(grid), dim3(kDThreads), 0, (hipStream_t)stream, codes,
                     (uint32_t)n_codes, bstart, n_elems, (const DictImage*)dict_image, dict_tag, out_fp16, bad,
                     (int)(((uintptr_t)codes & 15u) == 0));
  e = hipGetLastError();
  if (e != hipSuccess) return fail(SBM_EHIP, "decode_dense launch: %s", hipGetErrorString(e));
  return SBM_OK;
}
