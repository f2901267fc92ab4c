// Internal declarations shared by the host codec and the GPU entry points.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "sbm.h"

namespace sbm {

constexpr uint32_t kImageMagic = 0x53424D31u;  // "SBM1"
constexpr uint32_t kImageVersion = 5;
constexpr uint32_t kTabEntries = 15360;        // decode-table capacity: 60 KB
constexpr uint32_t kImage4Version = 6;
constexpr uint32_t kTab4Entries = 16768;       // 4-slot table capacity: 65.5 KB (p0 >= 0.857)

// Decode image of a dictionary (device copy read by the fused kernel): one
// 32-bit word per codeword says everything the kernel needs,
//   byte i (i = 0, 1, 2): 6*p_i + 2*[nonzero i is positive] for the i-th
//                         nonzero at run position p_i, or 4 when the entry has
//                         fewer than i+1 nonzeros (the byte offsets of the
//                         activation triple [-x, +x, 0] of a column);
//   byte 3:               6*L for a run of L symbols.
// The words are stored compressed.  From split H on every entry has 3
// nonzeros, and entries come in aligned groups of 8 that share positions and
// length and differ only in their signs: entry H + 8g + s has sign bit i of s
// for nonzero i (the canonical in-class order, colex rank * 8 + sign index).
// A group is stored once, without signs; entries below H are stored one by
// one.  With e = c + 7H:
//   idx(c)  = min(c, e >> 3)      (H + (c - H) / 8 from H on, at least c below)
//   word(c) = tab[idx(c)] + spread(e & 7),   spread(s) = ((s * 0x8102) & 0x20202)
// (e & 7 = (c - H) & 7; spread puts 2 * bit i of s into byte i).  Entries
// below H are stored as word(c) - spread(e & 7), so the same two steps
// rebuild every codeword.
struct DictImage {
  uint32_t magic;
  uint32_t version;
  uint32_t split;        // H
  uint32_t n_tab;        // used entries of tab: H + ceil((65536 - H) / 8)
  uint64_t checksum;
  uint64_t reserved1;
  uint32_t tab[kTabEntries];
};

// 4-slot decode image, for dictionaries whose entries hold up to 4 nonzeros
// (those built for P(0) below about 0.885 have runs of 4 nonzeros, all of
// length <= 14).  Same header and the same two steps with another word:
//   bits 7i .. 7i+6 (i = 0..3): k_i = 3*p_i + [nonzero i is positive] for the
//                         i-th nonzero at run position p_i, or 2 when the
//                         entry has fewer than i+1 nonzeros (2*k_i is the
//                         byte offset in the activation triples);
//   bits 28..31:          L / 2 (pairs in the run).
// From H on every entry has 3 or 4 nonzeros and groups of 8 share positions,
// length and the sign of a 4th nonzero (in-class rank = colex rank * 2^n +
// sign index, class sizes multiples of 8); spread(s) = ((s * 0x1041) & 0x4081)
// puts bit i of s into field i.
struct DictImage4 {
  uint32_t magic;
  uint32_t version;
  uint32_t split;
  uint32_t n_tab;
  uint64_t checksum;
  uint64_t reserved1;
  uint32_t tab[kTab4Entries];
};

int fail(int status, const char* fmt, ...);
const char* last_error();
int unpack(uint32_t w0, uint32_t w1, uint8_t* s);
int build_dictionary(double p0, uint32_t* words);
uint64_t checksum(const uint32_t* words);
int dict_image(const uint32_t* words, void* out, size_t bytes);
int dict_image4(const uint32_t* words, void* out, size_t bytes);
int build_trie(const uint32_t* words, std::vector<int32_t>& child);
int encode_size(const uint8_t* sym, int32_t rows, int32_t cols, const uint32_t* words,
                uint64_t* n_codes);
int encode_matrix(const uint8_t* sym, int32_t rows, int32_t cols, const uint32_t* words,
                  uint16_t* codes, uint64_t capacity, uint32_t* row_off, uint32_t* bstart,
                  uint64_t* n_codes);
int block_starts(const uint16_t* codes, uint64_t n, const uint32_t* words, uint32_t* bstart);
int encode_experts(int32_t n_mats, const uint8_t* const* sym, int32_t rows, int32_t cols,
                   const uint32_t* words, uint16_t* codes, uint64_t codes_capacity, uint32_t* row_off,
                   uint32_t* bstart, uint64_t bstart_capacity, sbm_matrix_desc* desc,
                   uint64_t* n_codes_total, uint64_t* n_blocks_total);
int validate_stream(const uint16_t* codes, uint64_t n, const uint32_t* row_off, int32_t rows,
                    int32_t cols, const uint32_t* words);
void div_magic(uint32_t d, uint64_t* m, uint32_t* shift);

}  // namespace sbm
