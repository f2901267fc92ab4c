// Host side of libsbm: dictionary construction, checksum, the compact decode
// image for the fused kernel, the greedy trie encoder, block offsets and
// stream validation.
//
// [QMoE] = "QMoE: Practical Sub-1-Bit Compression of Trillion-Parameter Models",
// sections "The Fixed-to-Variable Dictionary Code" (Algorithm 1, Eq. 2,
// Figure 4) and "The GPU Decoding Kernel" ("Encoding": trie, greedy longest
// prefix, rows independent, one offset per row).
#include "sbm_internal.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <unordered_map>
#include <vector>

namespace sbm {

static thread_local std::string g_err;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return status;
}

const char* last_error() { return g_err.c_str(); }

// ------------------------------------------------------------------ classes
// A class (L, n) holds every sequence of length L with n nonzero symbols; all
// have probability p0^(L-n) * q^n (Eq. 2).  Classes are ranked by that value,
// most probable first; values equal to 1e-9 (relative) are ties, ordered by
// shorter length, then fewer nonzeros.
struct Class {
  int L, n;
  double v;
};

static std::vector<Class> ranked_classes(double p0) {
  const double lp = std::log(p0), lq = std::log((1.0 - p0) / 2.0);
  std::vector<Class> cs;
  for (int L = 2; L <= SBM_MAX_RUN; L += 2)
    for (int n = 0; n <= L; ++n) cs.push_back({L, n, (L - n) * lp + n * lq});
  std::sort(cs.begin(), cs.end(), [](const Class& a, const Class& b) {
    const double tol = 1e-9 * std::max(1.0, std::max(std::fabs(a.v), std::fabs(b.v)));
    if (std::fabs(a.v - b.v) > tol) return a.v > b.v;
    if (a.L != b.L) return a.L < b.L;
    return a.n < b.n;
  });
  return cs;
}

// Next n-subset of {0..L-1} in colexicographic order; false after the last.
static bool colex_next(std::vector<int>& p, int L) {
  const int n = (int)p.size();
  for (int i = 0; i < n; ++i) {
    const int lim = (i + 1 < n) ? p[i + 1] : L;
    if (p[i] + 1 < lim) {
      ++p[i];
      for (int j = 0; j < i; ++j) p[j] = j;
      return true;
    }
  }
  return false;
}

static void pack(const uint8_t* s, int L, uint32_t* w) {
  const uint32_t k = (uint32_t)(L / 2);
  uint32_t w0 = k, w1 = k;
  for (int i = 0; i < L; ++i) {
    if (i < 14) w0 |= (uint32_t)s[i] << (4 + 2 * i);
    else w1 |= (uint32_t)s[i] << (4 + 2 * (i - 14));
  }
  w[0] = w0;
  w[1] = w1;
}

int unpack(uint32_t w0, uint32_t w1, uint8_t* s) {
  const uint32_t k = w0 & 0xF;
  if ((w1 & 0xF) != k || k < 1 || k > 14) return -1;
  const int L = (int)(2 * k);
  for (int i = 0; i < L; ++i) {
    const uint32_t w = i < 14 ? w0 : w1;
    const int j = i < 14 ? i : i - 14;
    s[i] = (uint8_t)((w >> (4 + 2 * j)) & 3u);
    if (s[i] == 3) return -1;
  }
  // slots past the pair count must be empty
  for (int i = L; i < 28; ++i) {
    const uint32_t w = i < 14 ? w0 : w1;
    const int j = i < 14 ? i : i - 14;
    if ((w >> (4 + 2 * j)) & 3u) return -1;
  }
  return L;
}

int build_dictionary(double p0, uint32_t* words) {
  if (!(p0 >= 0.5 && p0 < 1.0)) return fail(SBM_EINVAL, "p0 must lie in [0.5, 1)");
  const std::vector<Class> cs = ranked_classes(p0);
  uint32_t c = 0;
  uint8_t seq[SBM_MAX_RUN];
  for (const Class& k : cs) {
    if (c >= SBM_DICT_ENTRIES) break;
    std::vector<int> pos(k.n);
    for (int i = 0; i < k.n; ++i) pos[i] = i;
    bool more = true;
    while (more && c < SBM_DICT_ENTRIES) {
      for (uint32_t sg = 0; sg < (1u << k.n) && c < SBM_DICT_ENTRIES; ++sg) {
        std::memset(seq, 0, sizeof(seq));
        for (int i = 0; i < k.n; ++i) seq[pos[i]] = (sg >> i) & 1u ? 2 : 1;
        pack(seq, k.L, words + 2 * c);
        ++c;
      }
      more = colex_next(pos, k.L);
    }
  }
  if (c != SBM_DICT_ENTRIES) return fail(SBM_EDICT, "not enough candidate sequences");
  return SBM_OK;
}

uint64_t checksum(const uint32_t* words) {
  uint64_t h = 0xcbf29ce484222325ull;
  for (uint32_t i = 0; i < SBM_DICT_WORDS; ++i) {
    uint32_t w = words[i];
    for (int b = 0; b < 4; ++b) {
      h ^= (w >> (8 * b)) & 0xFFu;
      h *= 0x100000001b3ull;
    }
  }
  return h;
}

// ------------------------------------------------------------ decode image
static uint32_t spread3(uint32_t sg) { return ((sg & 7u) * 0x8102u) & 0x20202u; }

int dict_image(const uint32_t* words, void* out, size_t bytes) {
  if (!words || !out) return fail(SBM_EINVAL, "null pointer");
  if (bytes < sizeof(DictImage)) return fail(SBM_ENOSPACE, "image buffer too small");
  // the word of every codeword: slot bytes and 6 L; nonzero count and signs
  std::vector<uint32_t> word(SBM_DICT_ENTRIES);
  std::vector<uint8_t> nnz(SBM_DICT_ENTRIES), sidx(SBM_DICT_ENTRIES);
  uint8_t sym[SBM_MAX_RUN];
  for (uint32_t c = 0; c < SBM_DICT_ENTRIES; ++c) {
    const int L = unpack(words[2 * c], words[2 * c + 1], sym);
    if (L < 0) return fail(SBM_EDICT, "entry %u: malformed pair count or symbols", c);
    uint32_t w = (uint32_t)(6 * L) << 24, n = 0, sg = 0;
    for (int p = 0; p < L; ++p)
      if (sym[p]) {
        if (n >= 3) return fail(SBM_EDICT, "entry %u has more than 3 nonzeros", c);
        if (sym[p] == 2) sg |= 1u << n;
        w |= (uint32_t)(6 * p + (sym[p] == 2 ? 2 : 0)) << (8 * n);
        ++n;
      }
    for (uint32_t i = n; i < 3; ++i) w |= 4u << (8 * i);
    word[c] = w;
    nnz[c] = (uint8_t)n;
    sidx[c] = (uint8_t)sg;
  }
  // split: the first codeword from which on every entry has 3 nonzeros and
  // groups of 8 align (same positions and length, sign index = (c - H) & 7)
  uint32_t H = SBM_DICT_ENTRIES;
  while (H > 0 && nnz[H - 1] == 3) --H;
  auto aligned = [&](uint32_t h) {
    for (uint32_t c = h; c < SBM_DICT_ENTRIES; ++c) {
      const uint32_t s = (c - h) & 7u, c0 = c - s;
      if (sidx[c] != s || (word[c] - spread3(s)) != word[c0]) return false;
    }
    return true;
  };
  while (H < SBM_DICT_ENTRIES && !aligned(H)) ++H;
  const uint32_t n_tab = H + (SBM_DICT_ENTRIES - H + 7) / 8;
  if (n_tab > kTabEntries)
    return fail(SBM_EDICT, "dictionary needs %u decode-table entries (at most %u): fewer entries with 3 "
                           "nonzeros in aligned sign groups than the fused kernel assumes", n_tab, kTabEntries);
  DictImage* im = (DictImage*)out;
  std::memset(im, 0, sizeof(DictImage));
  im->magic = kImageMagic;
  im->version = kImageVersion;
  im->split = H;
  im->n_tab = n_tab;
  im->checksum = checksum(words);
  for (uint32_t c = 0; c < H; ++c) im->tab[c] = word[c] - spread3(c + 7 * H);
  for (uint32_t c = H; c < SBM_DICT_ENTRIES; c += 8) im->tab[H + (c - H) / 8] = word[c];
  // the kernel's two steps must rebuild every codeword's word
  for (uint32_t c = 0; c < SBM_DICT_ENTRIES; ++c) {
    const uint32_t e = c + 7 * H, idx = std::min(c, e >> 3);
    if (idx >= n_tab || im->tab[idx] + spread3(e) != word[c])
      return fail(SBM_EDICT, "internal: entry %u does not rebuild", c);
  }
  return SBM_OK;
}

// 4-slot image: 7-bit fields k = 3p + [positive] (2: empty), L / 2 on top.
static uint32_t spread4(uint32_t sg) { return ((sg & 7u) * 0x1041u) & 0x4081u; }

int dict_image4(const uint32_t* words, void* out, size_t bytes) {
  if (!words || !out) return fail(SBM_EINVAL, "null pointer");
  if (bytes < sizeof(DictImage4)) return fail(SBM_ENOSPACE, "image buffer too small");
  std::vector<uint32_t> word(SBM_DICT_ENTRIES);
  std::vector<uint8_t> nnz(SBM_DICT_ENTRIES), sidx(SBM_DICT_ENTRIES);
  uint8_t sym[SBM_MAX_RUN];
  for (uint32_t c = 0; c < SBM_DICT_ENTRIES; ++c) {
    const int L = unpack(words[2 * c], words[2 * c + 1], sym);
    if (L < 0) return fail(SBM_EDICT, "entry %u: malformed pair count or symbols", c);
    uint32_t w = (uint32_t)(L / 2) << 28, n = 0, sg = 0;
    for (int p = 0; p < L; ++p)
      if (sym[p]) {
        if (n >= 4) return fail(SBM_EDICT, "entry %u has more than 4 nonzeros", c);
        if (sym[p] == 2) sg |= 1u << n;
        w |= (uint32_t)(3 * p + (sym[p] == 2 ? 1 : 0)) << (7 * n);
        ++n;
      }
    for (uint32_t i = n; i < 4; ++i) w |= 2u << (7 * i);
    word[c] = w;
    nnz[c] = (uint8_t)n;
    sidx[c] = (uint8_t)sg;
  }
  // split: from H on every entry has 3 or 4 nonzeros, and groups of 8 align
  // (same word apart from the signs of nonzeros 0..2, which are (c - H) & 7)
  uint32_t H = SBM_DICT_ENTRIES;
  while (H > 0 && nnz[H - 1] >= 3) --H;
  auto aligned = [&](uint32_t h) {
    for (uint32_t c = h; c < SBM_DICT_ENTRIES; ++c) {
      const uint32_t s = (c - h) & 7u, c0 = c - s;
      if ((sidx[c] & 7u) != s || (word[c] - spread4(s)) != word[c0]) return false;
    }
    return true;
  };
  while (H < SBM_DICT_ENTRIES && !aligned(H)) ++H;
  const uint32_t n_tab = H + (SBM_DICT_ENTRIES - H + 7) / 8;
  if (n_tab > kTab4Entries)
    return fail(SBM_EDICT, "dictionary needs %u 4-slot decode-table entries (at most %u)", n_tab, kTab4Entries);
  DictImage4* im = (DictImage4*)out;
  std::memset(im, 0, sizeof(DictImage4));
  im->magic = kImageMagic;
  im->version = kImage4Version;
  im->split = H;
  im->n_tab = n_tab;
  im->checksum = checksum(words);
  for (uint32_t c = 0; c < H; ++c) im->tab[c] = word[c] - spread4(c + 7 * H);
  for (uint32_t c = H; c < SBM_DICT_ENTRIES; c += 8) im->tab[H + (c - H) / 8] = word[c];
  for (uint32_t c = 0; c < SBM_DICT_ENTRIES; ++c) {
    const uint32_t e = c + 7 * H, idx = std::min(c, e >> 3);
    if (idx >= n_tab || im->tab[idx] + spread4(e) != word[c])
      return fail(SBM_EDICT, "internal: entry %u does not rebuild", c);
  }
  return SBM_OK;
}

// ------------------------------------------------------------------ encoder
// Trie over pair extensions: child[node*9 + 3a+b] = codeword of the node's
// sequence extended by (a, b), or -1; node 65536 is the root (empty sequence).
static uint64_t seq_key(const uint8_t* s, int L) {
  uint64_t key = (uint64_t)L;
  for (int i = 0; i < L; ++i) key |= (uint64_t)s[i] << (5 + 2 * i);
  return key;
}

int build_trie(const uint32_t* words, std::vector<int32_t>& child) {
  std::unordered_map<uint64_t, int32_t> idx;
  idx.reserve(SBM_DICT_ENTRIES * 2);
  std::vector<uint8_t> all((size_t)SBM_DICT_ENTRIES * SBM_MAX_RUN);
  std::vector<int> len(SBM_DICT_ENTRIES);
  for (uint32_t c = 0; c < SBM_DICT_ENTRIES; ++c) {
    uint8_t* s = &all[(size_t)c * SBM_MAX_RUN];
    const int L = unpack(words[2 * c], words[2 * c + 1], s);
    if (L < 0) return fail(SBM_EDICT, "entry %u: malformed", c);
    len[c] = L;
    if (!idx.emplace(seq_key(s, L), (int32_t)c).second) return fail(SBM_EDICT, "duplicate entry %u", c);
  }
  child.assign((size_t)(SBM_DICT_ENTRIES + 1) * 9, -1);
  for (uint32_t c = 0; c < SBM_DICT_ENTRIES; ++c) {
    const uint8_t* s = &all[(size_t)c * SBM_MAX_RUN];
    const int L = len[c];
    // prefix closure: the entry must be reachable pair by pair from the root
    int32_t parent = SBM_DICT_ENTRIES;
    if (L > 2) {
      auto it = idx.find(seq_key(s, L - 2));
      if (it == idx.end()) return fail(SBM_EDICT, "entry %u: pair prefix missing (not prefix-closed)", c);
      parent = it->second;
    }
    child[(size_t)parent * 9 + 3 * s[L - 2] + s[L - 1]] = (int32_t)c;
  }
  for (int pr = 0; pr < 9; ++pr)
    if (child[(size_t)SBM_DICT_ENTRIES * 9 + pr] < 0) return fail(SBM_EDICT, "a single pair is missing");
  return SBM_OK;
}

// Greedy walk of one row; writes codes if out != nullptr.  Returns count.
static uint64_t encode_row(const uint8_t* row, int cols, const int32_t* child, uint16_t* out) {
  uint64_t n = 0;
  int pos = 0;
  while (pos < cols) {
    int32_t node = SBM_DICT_ENTRIES;
    int L = 0;
    while (pos + L + 2 <= cols && L + 2 <= SBM_MAX_RUN) {
      const int32_t nx = child[(size_t)node * 9 + 3 * row[pos + L] + row[pos + L + 1]];
      if (nx < 0) break;
      node = nx;
      L += 2;
    }
    if (out) out[n] = (uint16_t)node;
    ++n;
    pos += L;
  }
  return n;
}

static int check_matrix(const uint8_t* sym, int32_t rows, int32_t cols) {
  if (!sym && rows > 0) return fail(SBM_EINVAL, "null symbol matrix");
  if (rows < 0 || cols <= 0) return fail(SBM_EINVAL, "bad shape %d x %d", rows, cols);
  if (cols & 1) return fail(SBM_EODD_WIDTH, "cols=%d is odd", cols);
  const size_t total = (size_t)rows * (size_t)cols;
  for (size_t i = 0; i < total; ++i)
    if (sym[i] > 2) return fail(SBM_EINVAL, "symbol %u at %zu is not 0/1/2", sym[i], i);
  return SBM_OK;
}

static int n_threads_for(int32_t rows) {
  unsigned hw = std::thread::hardware_concurrency();
  int t = (int)std::min<unsigned>(hw ? hw : 1, 16);
  return std::max(1, std::min(t, rows / 64));
}

int encode_size(const uint8_t* sym, int32_t rows, int32_t cols, const uint32_t* words,
                uint64_t* n_codes) {
  if (!words || !n_codes) return fail(SBM_EINVAL, "null pointer");
  int st = check_matrix(sym, rows, cols);
  if (st) return st;
  std::vector<int32_t> child;
  if ((st = build_trie(words, child))) return st;
  std::vector<uint64_t> counts(rows);
  const int nt = n_threads_for(rows);
  std::vector<std::thread> th;
  for (int t = 0; t < nt; ++t)
    th.emplace_back([&, t] {
      for (int32_t r = t; r < rows; r += nt)
        counts[r] = encode_row(sym + (size_t)r * cols, cols, child.data(), nullptr);
    });
  for (auto& x : th) x.join();
  uint64_t n = 0;
  for (auto v : counts) n += v;
  *n_codes = n;
  return SBM_OK;
}

int encode_matrix(const uint8_t* sym, int32_t rows, int32_t cols, const uint32_t* words,
                  uint16_t* codes, uint64_t capacity, uint32_t* row_off, uint32_t* bstart,
                  uint64_t* n_codes) {
  if (!words || !row_off || !n_codes || (!codes && capacity)) return fail(SBM_EINVAL, "null pointer");
  int st = check_matrix(sym, rows, cols);
  if (st) return st;
  std::vector<int32_t> child;
  if ((st = build_trie(words, child))) return st;
  std::vector<uint64_t> counts(rows);
  const int nt = n_threads_for(rows);
  {
    std::vector<std::thread> th;
    for (int t = 0; t < nt; ++t)
      th.emplace_back([&, t] {
        for (int32_t r = t; r < rows; r += nt)
          counts[r] = encode_row(sym + (size_t)r * cols, cols, child.data(), nullptr);
      });
    for (auto& x : th) x.join();
  }
  uint64_t n = 0;
  row_off[0] = 0;
  for (int32_t r = 0; r < rows; ++r) {
    n += counts[r];
    if (n > 0xFFFFFFFFull) return fail(SBM_ERANGE, "more than 2^32-1 codewords in one matrix");
    row_off[r + 1] = (uint32_t)n;
  }
  *n_codes = n;
  if (n > capacity) return fail(SBM_ENOSPACE, "capacity %llu < %llu codewords",
                                (unsigned long long)capacity, (unsigned long long)n);
  {
    std::vector<std::thread> th;
    for (int t = 0; t < nt; ++t)
      th.emplace_back([&, t] {
        for (int32_t r = t; r < rows; r += nt)
          encode_row(sym + (size_t)r * cols, cols, child.data(), codes + row_off[r]);
      });
    for (auto& x : th) x.join();
  }
  if (bstart) return block_starts(codes, n, words, bstart);
  return SBM_OK;
}

// A whole projection in the fused kernel's stack layout: one trie for all
// matrices, every row counted first (sizes, offsets, aligned code bases),
// then encoded in place.
int encode_experts(int32_t n_mats, const uint8_t* const* sym, int32_t rows, int32_t cols,
                   const uint32_t* words, uint16_t* codes, uint64_t codes_capacity, uint32_t* row_off,
                   uint32_t* bstart, uint64_t bstart_capacity, sbm_matrix_desc* desc,
                   uint64_t* n_codes_total, uint64_t* n_blocks_total) {
  if (n_mats < 0 || (!sym && n_mats > 0) || !words || !n_codes_total || !n_blocks_total)
    return fail(SBM_EINVAL, "null pointer or negative matrix count");
  int st;
  for (int32_t i = 0; i < n_mats; ++i)
    if ((st = check_matrix(sym[i], rows, cols))) return st;
  std::vector<int32_t> child;
  if ((st = build_trie(words, child))) return st;
  const size_t R1 = (size_t)rows + 1;
  std::vector<uint32_t> offs((size_t)n_mats * R1);
  std::vector<uint64_t> base(n_mats), nc(n_mats), blk(n_mats);
  uint64_t total = 0, blocks = 0;
  const int nt = n_threads_for(rows);
  std::vector<uint64_t> counts(rows);
  for (int32_t i = 0; i < n_mats; ++i) {
    std::vector<std::thread> th;
    for (int t = 0; t < nt; ++t)
      th.emplace_back([&, t] {
        for (int32_t r = t; r < rows; r += nt)
          counts[r] = encode_row(sym[i] + (size_t)r * cols, cols, child.data(), nullptr);
      });
    for (auto& x : th) x.join();
    uint64_t n = 0;
    offs[i * R1] = 0;
    for (int32_t r = 0; r < rows; ++r) {
      n += counts[r];
      if (n > 0xFFFFFFFFull) return fail(SBM_ERANGE, "matrix %d: more than 2^32-1 codewords", i);
      offs[i * R1 + r + 1] = (uint32_t)n;
    }
    base[i] = total;
    nc[i] = n;
    blk[i] = blocks;
    total += n + ((SBM_CODE_ALIGN - n % SBM_CODE_ALIGN) % SBM_CODE_ALIGN);
    blocks += (n + SBM_BLOCK - 1) / SBM_BLOCK;
  }
  *n_codes_total = total;
  *n_blocks_total = blocks;
  if (!codes || !row_off || !bstart || !desc || total > codes_capacity || blocks > bstart_capacity)
    return fail(SBM_ENOSPACE, "stack needs %llu codewords and %llu block starts",
                (unsigned long long)total, (unsigned long long)blocks);
  std::copy(offs.begin(), offs.end(), row_off);
  const uint32_t tag = (uint32_t)checksum(words);   // the descriptors name their dictionary
  for (int32_t i = 0; i < n_mats; ++i) {
    uint16_t* out = codes + base[i];
    const uint32_t* off = offs.data() + i * R1;
    std::vector<std::thread> th;
    for (int t = 0; t < nt; ++t)
      th.emplace_back([&, t] {
        for (int32_t r = t; r < rows; r += nt)
          encode_row(sym[i] + (size_t)r * cols, cols, child.data(), out + off[r]);
      });
    for (auto& x : th) x.join();
    const uint64_t end = i + 1 < n_mats ? base[i + 1] : total;
    std::fill(out + nc[i], codes + end, (uint16_t)0);
    if ((st = block_starts(out, nc[i], words, bstart + blk[i]))) return st;
    desc[i].code_base = base[i];
    desc[i].off_base = (uint64_t)i * R1;
    desc[i].scale_base = (uint64_t)i * (uint64_t)rows;
    desc[i].blk_base = blk[i];
    desc[i].n_codes = (uint32_t)nc[i];
    desc[i].rows = rows;
    desc[i].cols = cols;
    desc[i].dict_tag = tag;
  }
  return SBM_OK;
}

int block_starts(const uint16_t* codes, uint64_t n, const uint32_t* words, uint32_t* bstart) {
  if ((!codes && n) || !words || (!bstart && n)) return fail(SBM_EINVAL, "null pointer");
  uint64_t pos = 0;
  for (uint64_t i = 0; i < n; ++i) {
    if (i % SBM_BLOCK == 0) {
      if (pos > 0xFFFFFFFFull) return fail(SBM_ERANGE, "block start exceeds 32 bits");
      bstart[i / SBM_BLOCK] = (uint32_t)pos;
    }
    const uint32_t k = words[2 * codes[i]] & 0xF;
    pos += 2 * k;
  }
  return SBM_OK;
}

int validate_stream(const uint16_t* codes, uint64_t n, const uint32_t* row_off, int32_t rows,
                    int32_t cols, const uint32_t* words) {
  if (!row_off || !words || (!codes && n)) return fail(SBM_EINVAL, "null pointer");
  if (rows < 0 || cols <= 0) return fail(SBM_EINVAL, "bad shape");
  if (cols & 1) return fail(SBM_EODD_WIDTH, "cols=%d is odd", cols);
  if (row_off[0] != 0) return fail(SBM_ECORRUPT, "row_off[0] != 0");
  if ((uint64_t)row_off[rows] != n) return fail(SBM_ECORRUPT, "row_off[rows]=%u != n=%llu",
                                                row_off[rows], (unsigned long long)n);
  for (int32_t r = 0; r < rows; ++r) {
    if (row_off[r + 1] < row_off[r]) return fail(SBM_ECORRUPT, "row_off decreases at row %d", r);
    uint64_t sum = 0;
    for (uint32_t i = row_off[r]; i < row_off[r + 1]; ++i) {
      const uint32_t k0 = words[2 * codes[i]] & 0xF, k1 = words[2 * codes[i] + 1] & 0xF;
      if (k0 != k1 || k0 == 0 || k0 > 14) return fail(SBM_EDICT, "codeword %u has a bad pair count", codes[i]);
      sum += 2 * k0;
    }
    if (sum != (uint64_t)cols)
      return fail(SBM_ECORRUPT, "row %d decodes to %llu symbols, expected %d", r,
                  (unsigned long long)sum, cols);
  }
  return SBM_OK;
}

// Magic multiplier for exact division of n < 2^30 by d (Granlund & Montgomery,
// "Division by invariant integers using multiplication", 1994, Thm 4.2):
// l = ceil(log2 d), m = floor(2^(30+l) / d) + 1, q = (n*m) >> (30+l).
void div_magic(uint32_t d, uint64_t* m, uint32_t* shift) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  *m = ((1ull << (30 + l)) / d) + 1;
  *shift = 30 + l;
}

}  // namespace sbm

// -------------------------------------------------------------- C entries
extern "C" {

const char* sbm_last_error(void) { return sbm::last_error(); }
const char* sbm_version(void) { return "sbm 0.1 gfx950"; }

int sbm_build_dictionary(double p0, uint32_t* out_words, uint64_t* out_checksum) {
  if (!out_words) return sbm::fail(SBM_EINVAL, "null out_words");
  int st = sbm::build_dictionary(p0, out_words);
  if (st) return st;
  if (out_checksum) *out_checksum = sbm::checksum(out_words);
  return SBM_OK;
}

int sbm_dictionary_checksum(const uint32_t* words, uint64_t* out_checksum) {
  if (!words || !out_checksum) return sbm::fail(SBM_EINVAL, "null pointer");
  *out_checksum = sbm::checksum(words);
  return SBM_OK;
}

size_t sbm_dict_image_bytes(void) { return sizeof(sbm::DictImage); }
size_t sbm_dict_image4_bytes(void) { return sizeof(sbm::DictImage4); }

int sbm_dict_image4(const uint32_t* words, void* out_image, size_t image_bytes) {
  return sbm::dict_image4(words, out_image, image_bytes);
}

int sbm_dict_image(const uint32_t* words, void* out_image, size_t image_bytes) {
  return sbm::dict_image(words, out_image, image_bytes);
}

size_t sbm_trie_words(void) { return (size_t)(SBM_DICT_ENTRIES + 1) * 9; }

int sbm_build_trie(const uint32_t* words, int32_t* out_child) {
  if (!words || !out_child) return sbm::fail(SBM_EINVAL, "null pointer");
  std::vector<int32_t> child;
  const int st = sbm::build_trie(words, child);
  if (st) return st;
  std::copy(child.begin(), child.end(), out_child);
  return SBM_OK;
}

int sbm_encode_size(const uint8_t* sym, int32_t rows, int32_t cols, const uint32_t* words,
                    uint64_t* n_codes) {
  return sbm::encode_size(sym, rows, cols, words, n_codes);
}

int sbm_encode_matrix(const uint8_t* sym, int32_t rows, int32_t cols, const uint32_t* words,
                      uint16_t* codes, uint64_t capacity, uint32_t* row_off, uint32_t* bstart,
                      uint64_t* n_codes) {
  return sbm::encode_matrix(sym, rows, cols, words, codes, capacity, row_off, bstart, n_codes);
}

int sbm_encode_experts(int32_t n_mats, const uint8_t* const* sym, int32_t rows, int32_t cols,
                       const uint32_t* words, uint16_t* codes, uint64_t codes_capacity, uint32_t* row_off,
                       uint32_t* bstart, uint64_t bstart_capacity, sbm_matrix_desc* desc,
                       uint64_t* n_codes_total, uint64_t* n_blocks_total) {
  return sbm::encode_experts(n_mats, sym, rows, cols, words, codes, codes_capacity, row_off, bstart,
                             bstart_capacity, desc, n_codes_total, n_blocks_total);
}

int sbm_block_starts(const uint16_t* codes, uint64_t n_codes, const uint32_t* words,
                     uint32_t* bstart) {
  return sbm::block_starts(codes, n_codes, words, bstart);
}

int sbm_validate_stream(const uint16_t* codes, uint64_t n_codes, const uint32_t* row_off,
                        int32_t rows, int32_t cols, const uint32_t* words) {
  return sbm::validate_stream(codes, n_codes, row_off, rows, cols, words);
}

}  // extern "C"
