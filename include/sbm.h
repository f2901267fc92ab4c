/*
 * sbm.h -- C ABI of libsbm: dictionary-coded ternary MoE expert weights,
 * decoded on the fly inside a fused decode + matrix-vector kernel on gfx950.
 *
 * Sources (by page title and section):
 *   [QMoE]  "QMoE: Practical Sub-1-Bit Compression of Trillion-Parameter
 *           Models", sections "The Fixed-to-Variable Dictionary Code"
 *           (Algorithm 1, Eq. 2, Figure 4) and "The GPU Decoding Kernel"
 *           (row offsets, ternary grid, fused decode-and-multiply, trie
 *           encoder, skipping experts without tokens).
 *   [M8.5]  "M8.5 - Extreme Weight Compression and Representations",
 *           0x08A (reference decoder: expand a row's codewords, map symbols
 *           through [zero, negative, positive]) and 0x08B (operator contract,
 *           codebook checksum).
 *
 * Conventions
 *   Symbols: 0 = zero, 1 = negative (w_min = -s_r), 2 = positive (+s_r).
 *   Dictionary: 65536 entries, entry c = words[2c] (pair count k in bits 0-3,
 *     symbol i in bits 4+2i, i = 0..13) and words[2c+1] (k again, symbols
 *     14..27).  Entries are ordered from most to least probable under the
 *     i.i.d. model P(0)=p0, P(1)=P(2)=(1-p0)/2; equally probable entries (same
 *     length and nonzero count) are ordered by the colexicographic rank of the
 *     nonzero positions, then by the sign index sum_i [symbol at p_i==2]*2^i.
 *   Encoded matrix (rows x cols, cols even):
 *     codes   uint16  row streams concatenated in row order (greedy longest
 *                     prefix, rows independent, no codeword spans two rows)
 *     row_off uint32  rows+1 matrix-local codeword offsets, row_off[0] = 0
 *     bstart  uint32  ceil(n_codes/SBM_BLOCK) entries: the linear symbol
 *                     position row*cols+col where codeword b*SBM_BLOCK starts
 *     scales  fp16    one per row (stored as uint16 bit patterns)
 *   Operator contract ([M8.5] 0x08A/0x08B): input fp16 (bf16 with
 *   SBM_F_IN_BF16); decoded operand
 *   ternary; fp32 accumulation; scale applied in fp32 in the epilogue; output
 *   fp16 or fp32.
 *
 * Ownership: the caller allocates and frees every buffer; the library keeps
 * no pointer after a call returns.  GPU calls are enqueued on the caller's
 * stream (a hipStream_t passed as void*; NULL = the null stream) and return
 * before the work completes.  Host-checkable errors return a negative status
 * synchronously and sbm_last_error() (thread-local) describes it.  Device
 * resident data (codes, offsets, ids) is trusted by the fused kernel, which
 * bounds every index it derives; out-of-range expert ids are skipped and
 * counted in the workspace error word.
 */
#ifndef SBM_H
#define SBM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SBM_DICT_ENTRIES 65536
#define SBM_DICT_WORDS   131072
#define SBM_MAX_RUN      28
#define SBM_BLOCK        1024     /* codewords per block-offset entry */
#define SBM_CODE_ALIGN   8        /* matrix code bases must be multiples of this */

typedef enum {
  SBM_OK = 0,
  SBM_EINVAL = -1,      /* null pointer, bad size or parameter */
  SBM_EODD_WIDTH = -2,  /* cols is odd: codewords expand to pairs */
  SBM_ECORRUPT = -3,    /* a code stream does not decode to its row widths */
  SBM_EDICT = -4,       /* dictionary is malformed or not in canonical order */
  SBM_ERANGE = -5,      /* a size exceeds what the layout can address */
  SBM_ENOSPACE = -6,    /* output capacity or workspace too small */
  SBM_EHIP = -7         /* a HIP runtime call failed (message in sbm_last_error) */
} sbm_status;

/* Flags of sbm_moe_fused_decode_matvec. */
#define SBM_F_RELU    1u  /* y = max(y, 0) after scaling (Switch experts are ReLU FFNs) */
#define SBM_F_OUT_F32 2u  /* y is float32 (default fp16) */
#define SBM_F_IN_RMS  4u  /* each x row is first scaled to unit RMS as sbm_rms_glue does (fp32
                             sum of squares, rounded to fp16); lets stacked layers skip that launch */
#define SBM_F_MFMA    8u  /* experts with 16 or more tokens take the dense-tile path: row tiles
                             decoded to a ternary tile in LDS, multiplied on the matrix cores
                             (v_mfma_f32_16x16x32_f16, fp32 accumulation).  Off by default: on
                             gfx950 it is slower than the sparse path up to 64 tokens per expert */
#define SBM_F_MINMAX 16u  /* [QMoE] "Quantization grid" and "The GPU Decoding Kernel": the per-row
                             grid {w_min, 0, w_max}.  scales then hold two fp16 per row, (w_min,
                             w_max) = the values of codes 1 and 2, at scales[scale_base + 2 r]
                             (scale_base even, scales 4-byte aligned); without it code 1 is -s_r
                             and code 2 is +s_r.  Each token is staged as two activation rows
                             ([-x, +x, 0] and [+x, +x, 0]) read at the same slot offsets, so an
                             item holds half as many tokens.  Not with SBM_F_MFMA. */
#define SBM_F_IMAGE4 32u  /* dict_image is a 4-slot image from sbm_dict_image4 (a dictionary built
                             for the data's P(0), whose entries may hold 4 nonzeros); the kernel
                             gathers 4 activation slots per codeword instead of 3, from a 65.5 KB
                             LDS table, which leaves less LDS for activation rows.  dict_image
                             must then hold sbm_dict_image4_bytes() bytes.  Not with SBM_F_MFMA. */
#define SBM_F_DETERMINISTIC 64u  /* bit-reproducible outputs: the row accumulators are 64-bit
                             integers in units of 2^-S (S = 34 - ceil(log2(3 (cols/1024 + 2))),
                             29 for 6144 columns) instead of fp32 LDS atomics, so each fp32
                             partial sum is rounded once to that grid and the sums do not depend
                             on the order in which waves add them.  The same call on the same
                             device then returns the same bits every time.  The pages leave the
                             summation order open.  Costs LDS (8-byte accumulators: shorter row
                             chunks) and a few conversions per block.  Activations must be finite.
                             Not with SBM_F_MFMA; not a flag of the layer call. */
#define SBM_F_IN_BF16 128u  /* x holds bf16 activations (the page's kernel reads bf16 x) instead of
                             fp16.  They are converted to fp16 as they are staged in LDS, which is
                             exact for magnitudes from 2^-14 to 65504 (smaller ones round to fp16
                             subnormals); |x| must stay below 65504.  With SBM_F_IN_RMS the RMS is
                             taken of the converted values.  Not with SBM_F_MFMA.  In the layer call
                             it applies to x (h stays fp16). */

/* Thread-local text of the last non-OK status returned on this thread. */
const char* sbm_last_error(void);
const char* sbm_version(void);

/* ------------------------------------------------------------ dictionary */

/* [QMoE] Algorithm 1 / Figure 4: the canonical 65536-entry dictionary for
 * zero probability p0 (0.5 <= p0 < 1; the page's static table uses 0.885).
 * out_words: host, SBM_DICT_WORDS uint32.  out_checksum (may be NULL):
 * FNV-1a 64 over the words' little-endian bytes. */
int sbm_build_dictionary(double p0, uint32_t* out_words, uint64_t* out_checksum);

/* FNV-1a 64 of the 512 KB packed table (the [M8.5] 0x08B codebook checksum). */
int sbm_dictionary_checksum(const uint32_t* words, uint64_t* out_checksum);

/* Compact decode image for the fused kernel (one 32-bit word per codeword:
 * nonzero positions, signs and run length), derived from a dictionary in
 * which every entry has at most 3 nonzeros and, from some split codeword H
 * on, every entry has exactly 3, in aligned groups of 8 that differ only in
 * their signs (sign bit i of (c - H) & 7 for nonzero i: the canonical order
 * above), with H + (65536 - H) / 8 at most 15360 table words.  Host in, host
 * out; the caller uploads the image to the device.  Returns SBM_EDICT if the
 * dictionary does not have that structure. */
size_t sbm_dict_image_bytes(void);
int sbm_dict_image(const uint32_t* words, void* out_image, size_t image_bytes);

/* [QMoE] "Limitations and Trade-offs" (the dictionary is static, tuned to
 * c2048's P(0); a table per model is the suggested remedy) and Table 7: the
 * decode image of a dictionary built for other data.  Tables built for p0
 * below ~0.885 hold entries with 4 nonzeros (all in runs of at most 14
 * symbols).  Word per codeword: four 7-bit slots k = 3p + [positive] (2 when
 * empty) and L / 2 in the top 4 bits; from a split H on, every entry has 3 or
 * 4 nonzeros in aligned groups of 8 that differ only in the signs of their
 * first three nonzeros, stored once.  Requires at most 4 nonzeros per entry
 * and H + (65536 - H) / 8 <= 16768 table words: canonical tables for
 * 0.857 <= p0 < 1, which covers the sparsities the page reports for base128,
 * large128 and c2048 (85.7%, 86.4%, 88.6%).  Host in, host out; SBM_EDICT
 * otherwise.  Use the image with SBM_F_IMAGE4. */
size_t sbm_dict_image4_bytes(void);
int sbm_dict_image4(const uint32_t* words, void* out_image, size_t image_bytes);

/* ----------------------------------------------------------- host codec */

/* [QMoE] "Encoding": greedy longest-prefix walk of each row over a trie of the
 * dictionary.  sym: host uint8 [rows x cols] row-major, values 0/1/2.
 * Size query: n_codes receives the number of codewords. */
int sbm_encode_size(const uint8_t* sym, int32_t rows, int32_t cols,
                    const uint32_t* words, uint64_t* n_codes);

/* Fill codes (capacity entries), row_off (rows+1) and, if bstart is not NULL,
 * the ceil(n/SBM_BLOCK) block start positions.  n_codes receives the count. */
int sbm_encode_matrix(const uint8_t* sym, int32_t rows, int32_t cols,
                      const uint32_t* words, uint16_t* codes, uint64_t capacity,
                      uint32_t* row_off, uint32_t* bstart, uint64_t* n_codes);

/* Block start positions of an existing stream (host). */
int sbm_block_starts(const uint16_t* codes, uint64_t n_codes, const uint32_t* words,
                     uint32_t* bstart);

/* Host check that every row of a stream decodes to exactly cols symbols and
 * that row_off is monotone and ends at n_codes.  SBM_ECORRUPT otherwise. */
int sbm_validate_stream(const uint16_t* codes, uint64_t n_codes, const uint32_t* row_off,
                        int32_t rows, int32_t cols, const uint32_t* words);

/* -------------------------------------------------------------- GPU path */

/* One matrix of an expert stack, as the fused kernel sees it (device table). */
typedef struct {
  uint64_t code_base;   /* first codeword in `codes` (multiple of SBM_CODE_ALIGN) */
  uint64_t off_base;    /* first of the matrix's rows+1 entries in `row_off` */
  uint64_t scale_base;  /* first of the matrix's `rows` entries in `scales` (2 rows entries with
                           SBM_F_MINMAX) */
  uint64_t blk_base;    /* first of the matrix's block starts in `bstart` */
  uint32_t n_codes;     /* codewords of the matrix */
  int32_t rows;
  int32_t cols;
  uint32_t dict_tag;    /* identity of the dictionary the codes were encoded with: the low 32 bits of
                           its FNV-1a 64 checksum ([M8.5] 0x08B: the codebook checksum belongs to the
                           artefact, since a reordered codebook corrupts every index).  The fused
                           kernel and the dense decoder compare it with the decode image's checksum
                           and refuse the matrix on a mismatch. */
} sbm_matrix_desc;

/* [QMoE] "Encoding" for a whole projection (host): n_mats matrices of one
 * shape, sym[i] host uint8 [rows x cols] with values 0/1/2, encoded into one
 * stack in the layout sbm_moe_fused_decode_matvec reads:
 *   codes:   every matrix's codewords from a base that is a multiple of
 *            SBM_CODE_ALIGN, the gaps zero (codes_capacity entries);
 *   row_off: n_mats * (rows + 1) matrix-local offsets;
 *   bstart:  every matrix's ceil(n/SBM_BLOCK) block starts, concatenated
 *            (bstart_capacity entries);
 *   desc:    host sbm_matrix_desc[n_mats], scale_base = i * rows (the caller
 *            lays out the scales, one or two fp16 per row in matrix order;
 *            double scale_base for SBM_F_MINMAX), dict_tag = the low 32 bits
 *            of the FNV-1a 64 checksum of `words`.
 * n_codes_total and n_blocks_total always receive the sizes needed; with a
 * NULL output or a capacity below them the call returns SBM_ENOSPACE after
 * writing them (the size query).  The trie is built once for all matrices. */
int sbm_encode_experts(int32_t n_mats, const uint8_t* const* sym, int32_t rows, int32_t cols,
                       const uint32_t* words, uint16_t* codes, uint64_t codes_capacity, uint32_t* row_off,
                       uint32_t* bstart, uint64_t bstart_capacity, sbm_matrix_desc* desc,
                       uint64_t* n_codes_total, uint64_t* n_blocks_total);

/* Decompression for the two-launch path ([QMoE] "The GPU Decoding Kernel":
 * decompress, then multiply, is what the fused kernel avoids): one matrix to
 * dense row-major fp16 values -1, 0, +1 (the row scale is left for the GEMM's
 * epilogue, so the output is exact).  codes: device, the matrix's n_codes
 * codewords (n_codes >= 1, < 2^32); bstart: device, its ceil(n_codes/SBM_BLOCK)
 * block starts; dict_image: device copy of sbm_dict_image() output;
 * out_fp16: device [rows x cols], 4-byte aligned, every element written;
 * bad: device uint32 set to 1 if the image fails its header check (then
 * nothing is written; the caller zeroes it beforehand) and set to 2 if
 * dict_tag (the matrix descriptor's dictionary tag) differs from the low 32
 * bits of the image's dictionary checksum (nothing is written either).
 * rows * cols < 2^32, cols even.  One wave per 1024-codeword block: coalesced
 * zero-fill of the block's element span (16-byte stores where out is 16-byte
 * aligned), the block's codewords (16-byte loads when codes is 16-byte
 * aligned) looked up in the image's table, then a store per nonzero. */
int sbm_decode_dense(const uint16_t* codes, uint64_t n_codes, const uint32_t* bstart, int32_t rows,
                     int32_t cols, const void* dict_image, uint32_t dict_tag, uint16_t* out_fp16, uint32_t* bad,
                     void* stream);

/* [M8.5] 0x08A reference decode on the GPU: one matrix to symbols.
 * codes, row_off, words, out_sym: device.  out_sym: uint8 [rows x cols].
 * One thread per row expands its codewords from the packed words; a row whose
 * stream does not total cols symbols is written as far as it goes and the
 * count of such rows is added to *bad_rows (device uint32, may be NULL). */
int sbm_decode_ref(const uint16_t* codes, const uint32_t* row_off, int32_t rows, int32_t cols,
                   const uint32_t* words, uint8_t* out_sym, uint32_t* bad_rows, void* stream);

/* Workspace bytes needed by sbm_moe_fused_decode_matvec. */
size_t sbm_workspace_bytes(int32_t n_experts, int32_t n_tokens);

/* [QMoE] "The GPU Decoding Kernel", grouped over experts: for every token t,
 *   y[t, r] = act( sum_j W_e[r, j] * x[t, j] ),  e = expert_ids[t],
 * where W_e is expert e's ternary matrix on its per-row grid (codes 1, 2 ->
 * -s_r, +s_r, or w_min, w_max with SBM_F_MINMAX) (rows x cols, the same shape for all
 * experts of the call) decoded from its code stream without materialising it.
 * Experts without tokens are skipped.  Tokens with an id outside [0, n_experts)
 * produce no output row and are counted in the workspace error word; so are
 * tokens routed to an expert whose descriptor disagrees with the call (shape,
 * alignment) or whose dict_tag differs from the image's dictionary checksum:
 * those produce no output row either, and set bits 30 / 29 of that word.
 *   codes/row_off/bstart/scales: device arrays addressed through `experts`;
 *               a matrix's codes are read in whole dwords (after an odd count,
 *               the 2 bytes sharing the last codeword's dword are read and ignored)
 *   experts:    device sbm_matrix_desc[n_experts] (dict_tag = the image's dictionary)
 *   dict_image: device copy of sbm_dict_image() output (sbm_dict_image4() with SBM_F_IMAGE4);
 *               an image of the other kind, or a damaged one, sets the workspace error word
 *   x:          device fp16 (bf16 with SBM_F_IN_BF16) [n_tokens x cols];  expert_ids: device int32 [n_tokens]
 *   y:          device [n_tokens x rows], fp16 (or fp32 with SBM_F_OUT_F32)
 *   workspace:  device, at least sbm_workspace_bytes(n_experts, n_tokens)
 * n_tokens may be 0 (nothing is launched).  cols must be even, 2..65536;
 * rows 1..2^24; rows*cols*6 < 2^30. */
int sbm_moe_fused_decode_matvec(const uint16_t* codes, const uint32_t* row_off,
                                const uint32_t* bstart, const uint16_t* scales,
                                const sbm_matrix_desc* experts, int32_t n_experts,
                                int32_t rows, int32_t cols, const void* dict_image,
                                const uint16_t* x, const int32_t* expert_ids, int32_t n_tokens,
                                void* y, uint32_t flags, void* workspace, size_t workspace_bytes,
                                void* stream);

/* One projection (all experts' matrices of one shape) of an MoE layer, as
 * the layer call reads it: the arrays and descriptor table described at
 * sbm_moe_fused_decode_matvec. */
typedef struct {
  const uint16_t* codes;
  const uint32_t* row_off;
  const uint32_t* bstart;
  const uint16_t* scales;
  const sbm_matrix_desc* experts;  /* device, [n_experts] */
  int32_t n_experts;
  int32_t rows;
  int32_t cols;
} sbm_projection;

/* Workspace bytes of sbm_moe_fused_ffn. */
size_t sbm_ffn_workspace_bytes(int32_t n_experts, int32_t n_tokens);

/* [QMoE] "The GPU Decoding Kernel" for a whole expert FFN in one launch: for
 * every token t with e = expert_ids[t],
 *   h[t, :] = relu( W_up_e x[t, :] )          (fp16, up: rows = f, cols = d)
 *   y[t, :] = W_down_e h[t, :]                (down: rows = d', cols = f)
 * on the per-row ternary grid (codes 1, 2 -> -s_r, +s_r), both projections
 * decoded on the fly as in sbm_moe_fused_decode_matvec.  The down rows of a
 * token start once all of its up rows are written (per-token counts in the
 * workspace; h is written and read coherently at device scope), so a layer
 * takes one launch instead of two (with more than 128 tokens, after a
 * grouping launch).  up, down: host structs of device arrays
 * with the same experts; up->rows == down->cols; both cols even and >= 512
 * (narrower rows: two sbm_moe_fused_decode_matvec calls).  x: device fp16
 * (bf16 with SBM_F_IN_BF16) [n_tokens x up->cols]; h: device fp16
 * [n_tokens x up->rows] (written);
 * y: device [n_tokens x down->rows], fp16 or fp32 (SBM_F_OUT_F32); x, h and y
 * must not overlap (workgroups still reading x run beside others writing y).  flags:
 * SBM_F_IN_RMS, SBM_F_OUT_F32, SBM_F_IN_BF16 only (symmetric grid, 3-slot
 * image).
 * workspace: device, 16-byte aligned, sbm_ffn_workspace_bytes(n_experts,
 * n_tokens) bytes, ZEROED by the caller before its first use with a call;
 * every call leaves it ready for the next (calls sharing a workspace must not
 * overlap).  Its first word is the call's error word (sbm_workspace_error),
 * as for sbm_moe_fused_decode_matvec, plus bit 28: the down phase gave up
 * waiting for up rows (about 20 ms, e.g. when not every workgroup could be
 * resident, or the workspace was not zeroed): those tokens' y is invalid. */
int sbm_moe_fused_ffn(const sbm_projection* up, const sbm_projection* down, const void* dict_image,
                      const uint16_t* x, const int32_t* expert_ids, int32_t n_tokens, uint16_t* h, void* y,
                      uint32_t flags, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of sbm_moe_fused_layers. */
size_t sbm_layers_workspace_bytes(int32_t n_layers, int32_t n_experts, int32_t n_tokens);

/* [QMoE] "The GPU Decoding Kernel" for n_layers MoE layers in one layer launch: for
 * l = 0 .. n_layers-1 and every token t with e = expert_ids[l * n_tokens + t],
 *   x_0 = x,  x_l = y_{l-1} / rms(y_{l-1}) per token for l >= 1
 *   h[t, :]   = relu( W_up_{l,e} x_l[t, :] )
 *   y_l[t, :] = W_down_{l,e} h[t, :]
 * as sbm_moe_fused_ffn computes each layer (the RMS scaling between layers is
 * the one SBM_F_IN_RMS applies; with the flag, layer 0's input is scaled too).
 * Every layer's routing is an input.  A workgroup prepares each projection
 * (chunk table, first code blocks) while the previous one is still finishing
 * elsewhere, and starts a token's rows as soon as that token's input rows are
 * all written.  The tokens of every projection are grouped by a short launch
 * before the layer launch (with one layer and at most 128 tokens, inside the
 * layer launch instead), all on `stream`.  up, down: arrays of n_layers host
 * structs (1 <= n_layers <= 32; longer stacks: one call per 32 layers), all
 * layers of layer 0's shapes, up->rows == down->cols and down->rows ==
 * up->cols when n_layers > 1, cols even and >= 512.  expert_ids: device int32
 * [n_layers x n_tokens].  x: device fp16 (bf16 with SBM_F_IN_BF16, layer 0
 * only) [n_tokens x up->cols]; h: device fp16 [n_layers x n_tokens x
 * up->rows] (written: every layer's h); y: device fp16 [n_layers x n_tokens x
 * down->rows] (written: every layer's output, the last layer's last).  x, h
 * and y must not overlap.  flags: SBM_F_IN_RMS, SBM_F_IN_BF16 (SBM_F_OUT_F32 with
 * n_layers = 1 only).  workspace: device, 16-byte aligned,
 * sbm_layers_workspace_bytes(n_layers, n_experts, n_tokens) bytes, ZEROED by
 * the caller before its first use with a call; every call leaves it ready for
 * the next (calls sharing a workspace must not overlap).  Its first word is
 * the call's error word as for sbm_moe_fused_ffn (invalid ids counted once
 * per layer; bit 28: a projection gave up waiting for its input rows).  With
 * n_layers = 1 this is sbm_moe_fused_ffn. */
int sbm_moe_fused_layers(const sbm_projection* up, const sbm_projection* down, int32_t n_layers,
                         const void* dict_image, const uint16_t* x, const int32_t* expert_ids, int32_t n_tokens,
                         uint16_t* h, uint16_t* y, uint32_t flags, void* workspace, size_t workspace_bytes,
                         void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * fused call with no workspace argument.  The kernels use a static device
 * array of 256 KiB (one copy per GPU the library runs on, held until the
 * process ends) in place of the workspace; calls whose
 * sbm_workspace_bytes(n_experts, n_tokens) exceeds it return SBM_ERANGE and
 * launch nothing.  The call allocates nothing and leaves no state that a
 * later call relies on.  Calls that overlap on one GPU (other streams, other
 * host threads) share that array and race: serialise them.  error_word:
 * device uint32 that receives the error word described at
 * sbm_workspace_error (may be NULL).  Every other argument as for
 * sbm_moe_fused_decode_matvec. */
int sbm_moe_fused_decode_matvec_noalloc(const uint16_t* codes, const uint32_t* row_off,
                                        const uint32_t* bstart, const uint16_t* scales,
                                        const sbm_matrix_desc* experts, int32_t n_experts,
                                        int32_t rows, int32_t cols, const void* dict_image,
                                        const uint16_t* x, const int32_t* expert_ids, int32_t n_tokens,
                                        void* y, uint32_t flags, uint32_t* error_word, void* stream);

/* ------------------------------------------- synthetic stack generation */
/* The QMoE page's c2048 stack (1.6T parameters, under 160 GB at ~0.8 bit per
 * parameter, ~88.6% zeros; Executive Summary and "Natural sparsity") cannot be
 * held as ternary symbols, so benchmark stacks are generated on the GPU row by
 * row and encoded on the fly with the same greedy trie walk as the host
 * encoder.  Symbols come from SplitMix64 (Steele, Lea, Flood 2014) used as a
 * counter-based generator:
 *   out(s, i)  = mix64(s + i * 0x9E3779B97F4A7C15)
 *   key        = out(seed, m + 1),  m = (layer * n_experts + expert) * 2 + mat
 *   symbol r,j = 16-bit lane j%4 of out(key, r*ceil(cols/4) + j/4 + 1):
 *                v < zero_threshold16 -> 0, odd v -> 2 (+), even v -> 1 (-)
 *   scale r    = scale_table[out(key, 2^40 + r + 1) >> 52]  (4096 fp16 entries)
 * mat 0 = up projection, 1 = down projection.  All buffers are device memory
 * owned by the caller. */

/* Trie child table of a dictionary: (SBM_DICT_ENTRIES+1)*9 int32; entry
 * node*9 + 3a+b is the codeword of node's sequence extended by pair (a,b), or
 * -1; node SBM_DICT_ENTRIES is the empty sequence.  Host in, host out. */
size_t sbm_trie_words(void);
int sbm_build_trie(const uint32_t* words, int32_t* out_child);

/* Pass 1: codeword count of every row of n_experts matrices -> row_counts[E*rows]. */
int sbm_gen_count(uint64_t seed, int32_t layer, int32_t n_experts, int32_t mat, int32_t rows, int32_t cols,
                  uint32_t zero_threshold16, const int32_t* trie, uint32_t* row_counts, void* stream);

/* Row offsets (E*(rows+1), matrix-local), matrix descriptors (E) and totals
 * (uint64[2]: codewords including per-matrix alignment padding, blocks).
 * dict_checksum: FNV-1a 64 checksum of the dictionary the trie was built
 * from (its low 32 bits become every descriptor's dict_tag). */
int sbm_gen_layout(const uint32_t* row_counts, int32_t n_experts, int32_t rows, int32_t cols, uint32_t* row_off,
                   sbm_matrix_desc* desc, uint64_t* totals, uint64_t dict_checksum, void* stream);

/* Pass 2: codewords, block starts and row scales into arrays sized from totals. */
int sbm_gen_write(uint64_t seed, int32_t layer, int32_t n_experts, int32_t mat, int32_t rows, int32_t cols,
                  uint32_t zero_threshold16, const int32_t* trie, const uint32_t* row_off,
                  const sbm_matrix_desc* desc, uint16_t* codes, uint32_t* bstart, const uint16_t* scale_table,
                  uint16_t* scales, void* stream);

/* Benchmark glue between stacked layers (not part of the method): per token,
 * x_out = y / sqrt(mean(y^2)) in fp32, stored fp16.  y, x_out: device fp16
 * [n_tokens x d]; they may not alias. */
int sbm_rms_glue(const uint16_t* y, int32_t n_tokens, int32_t d, uint16_t* x_out, void* stream);

/* Bandwidth probe (not part of the method): the cache-amplification page
 * measures a GPU device copy as the practical ceiling of its host roofline
 * ("Results", host roofline).  Streams `bytes` (a multiple of 16, buf 16-byte
 * aligned) of device memory through 16-byte loads in a grid of at most
 * sink_words workgroups, each writing one folded word to device sink[]; time
 * the call on `stream` to get the read bandwidth. */
int sbm_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, uint32_t sink_words, void* stream);

/* Workspace error word of the last fused call (device read; synchronises the
 * stream).  Bits 0-27: number of tokens whose expert id was out of range;
 * bit 28: (layer calls) the down phase gave up waiting for up rows;
 * bit 29: a touched expert's dict_tag differs from the image's dictionary
 * checksum (its tokens get no output); bit 30: a touched expert's descriptor
 * disagrees with the call's shape or alignment (its tokens get no output);
 * bit 31: the decode image failed its header check (nothing was computed). */
int sbm_workspace_error(const void* workspace, uint32_t* out_error, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SBM_H */
