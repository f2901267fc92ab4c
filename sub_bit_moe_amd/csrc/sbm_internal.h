// Internal declarations shared by the host codec and the GPU entry points.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "sbm.h"

namespace sbm {

constexpr uint32_t kImageMagic = 0x53424D31u;  // "SBM1"
constexpr uint32_t kImageVersion = 4;
constexpr int kMaxClasses = 64;

// Position table segments: colex-ordered n-subsets of {0..27} for n = 0..3.
// For a class of length L every rank below C(L, n) names a subset of {0..L-1},
// because colex order lists the subsets of a smaller ground set first.
constexpr uint32_t kPostSeg0 = 0;
constexpr uint32_t kPostSeg1 = 1;
constexpr uint32_t kPostSeg2 = 29;
constexpr uint32_t kPostSeg3 = 407;
constexpr uint32_t kPostEntries = 3683;

// Compact decode image of a canonical dictionary (device copy read by the
// fused kernel).  Codeword c of class k (cls_base[k] <= c < cls_base[k+1],
// n(k) nonzeros, length L(k)):
//   off   = c + K(k),  K(k) = seg(n) * 2^n - cls_base[k]
//   pidx  = off >> n                    (seg(n) + colex rank of the positions)
//   sg    = off & 7                     (bit i < n set: nonzero i is positive)
//   slots = postab[pidx] + spread(sg)
// Adding a multiple of 2^n keeps the sign bits of the in-class offset and
// moves the colex rank into the class's position-table segment.  spread puts
// 2*bit i of sg into byte i.  Byte i of a slot word is the byte offset
// 6*p_i + 2*positive of nonzero i in the [-x, +x, 0] triple layout, or 4 (the
// zero) when i >= n.  For i >= n, bit i of off is bit i - n of pidx, so those
// postab bytes are stored as 4 - 2*bit_{i-n}(pidx), which the spread brings
// back to 4.
// ctab[k] = (K(k) & 0x1FFFF) | n << 17 | (6*L) << 24   (K: 17-bit two's complement)
// cls[c]  = 4*k                                          (byte offset of ctab[k])
struct DictImage {
  uint32_t magic;
  uint32_t version;
  uint32_t n_classes;
  uint32_t reserved0;
  uint64_t checksum;
  uint64_t reserved1;
  uint32_t cls_base[kMaxClasses + 4];
  uint32_t ctab[kMaxClasses];
  uint32_t postab[kPostEntries + 1];
  uint8_t cls[SBM_DICT_ENTRIES];    // 4 * class of every codeword
};

int fail(int status, const char* fmt, ...);
const char* last_error();
int unpack(uint32_t w0, uint32_t w1, uint8_t* s);
int build_dictionary(double p0, uint32_t* words);
uint64_t checksum(const uint32_t* words);
int dict_image(const uint32_t* words, void* out, size_t bytes);
int build_trie(const uint32_t* words, std::vector<int32_t>& child);
int encode_size(const uint8_t* sym, int32_t rows, int32_t cols, const uint32_t* words,
                uint64_t* n_codes);
int encode_matrix(const uint8_t* sym, int32_t rows, int32_t cols, const uint32_t* words,
                  uint16_t* codes, uint64_t capacity, uint32_t* row_off, uint32_t* bstart,
                  uint64_t* n_codes);
int block_starts(const uint16_t* codes, uint64_t n, const uint32_t* words, uint32_t* bstart);
int validate_stream(const uint16_t* codes, uint64_t n, const uint32_t* row_off, int32_t rows,
                    int32_t cols, const uint32_t* words);
void div_magic(uint32_t d, uint64_t* m, uint32_t* shift);

}  // namespace sbm
