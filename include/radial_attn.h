/*
 * radial_attn.h — C ABI of libradial.so: Radial Attention forward pass on gfx950.
 *
 * The operation, after these pages:
 *  - "Radial Attention: O(n log n) Sparse Attention with Energy Decay for Long Video
 *    Generation" (paper summary page), Outline. Softmax attention over a video token
 *    sequence, where each query attends to spatially close keys and the window narrows
 *    as the temporal distance grows.
 *  - "Radial Attention: A Breakthrough in Efficient Long Video Generation", How Radial
 *    Attention Works. The mask is static, compute density halves when temporal distance
 *    doubles, and the mask is applied in 128x128 blocks.
 *  - The radial-attention-video SKILL.md page, Step 1 and Step 2. Tokens are frame-major
 *    (frame = t / S, spatial = t % S), masked scores are -inf before the softmax, and
 *    out = softmax(Q K^T * scale) V with one mask for every batch and head.
 *
 * The rule this library implements, with W0 the base spatial window:
 *     key k allowed for query q  <=>  |s_q - s_k| * 2^floor(log2(|f_q - f_k| + 1)) < W0
 * A 128x128 block is active iff it contains at least one allowed (query, key) pair.
 * Every real key of an active block takes part in that query block's softmax.
 * Variants: element masking (the rule applied to single entries inside the active
 * blocks, evaluated in the kernels or read from an element table built once per mask),
 * the 2-D grid distance (frames as grids of rows, |s_q - s_k| replaced by the Manhattan
 * distance between grid positions), a mask derived in the kernel instead of read from a
 * CSR, a packed batch of videos of different lengths, and the backward pass.
 *
 * Conventions for every call:
 *  - The return value is 0 (RADIAL_OK) on success or a negative RADIAL_ERR_* code.
 *    No call aborts or prints.
 *  - All buffers are owned by the caller. The library allocates no device memory. Its
 *    only state is described under radial_attn_fwd (work counters in static device
 *    memory and the events that guard their reuse).
 *  - Every check that can fail is done on the host before any HIP call.
 */
#ifndef RADIAL_ATTN_H
#define RADIAL_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  RADIAL_OK = 0,
  RADIAL_ERR_INVALID_ARG = -1,          /* a size <= 0, block != 128, null pointer, bad scale */
  RADIAL_ERR_UNSUPPORTED_HEAD_DIM = -2, /* head_dim other than 64 or 128 */
  RADIAL_ERR_CAPACITY = -3,             /* nnz_capacity smaller than the mask needs */
  RADIAL_ERR_SHAPE_MISMATCH = -4,       /* nb != ceil(seqlen / 128) */
  RADIAL_ERR_MISALIGNED = -5,           /* pointer or stride not a multiple of 16 bytes */
  RADIAL_ERR_TOO_LARGE = -6,            /* a count past the int32 index range */
  RADIAL_ERR_HIP = -7                   /* the HIP runtime reported an error at launch */
};

/* Block size of the mask in tokens, on both axes. */
#define RADIAL_BLOCK 128

/*
 * radial_mask_dims — sizes of the block mask for a video of `frames` x `tokens_per_frame`
 * tokens with base window `w0`. The mask is the static radial mask of "Radial Attention:
 * A Breakthrough in Efficient Long Video Generation", How Radial Attention Works (the
 * spatial window halves each time the temporal distance doubles, applied in 128x128
 * blocks), with frame-major tokens as on the radial-attention-video SKILL.md page,
 * Step 1; the rule is the one stated at the top of this header. It writes the number of
 * block rows nb = ceil(frames * tokens_per_frame / 128) to *nb_out, and the number of
 * active blocks to *nnz_out. It runs on the host only.
 *
 * Errors: INVALID_ARG if frames, tokens_per_frame or w0 is <= 0, if block != 128, or if
 * an output pointer is null. TOO_LARGE if the sequence length or the active-block count
 * does not fit in int32.
 */
int32_t radial_mask_dims(int32_t frames, int32_t tokens_per_frame, int32_t w0, int32_t block,
                         int32_t* nb_out, int64_t* nnz_out);

/*
 * radial_build_mask — fill the block mask of radial_mask_dims (the same pages: a block is
 * active iff one of its (query, key) pairs passes the rule) in compressed-row form. This
 * is host code and is deterministic.
 *
 * row_ptr: caller-owned host array of nb + 1 int32. row_ptr[0] = 0, and row r's active key
 *          blocks are col_idx[row_ptr[r] .. row_ptr[r+1]).
 * col_idx: caller-owned host array of at least nnz_capacity int32. Within each row the
 *          indices are strictly ascending, so a mask has exactly one such form.
 * Arguments and errors are as for radial_mask_dims, plus CAPACITY when nnz_capacity is
 * smaller than the active-block count. On any error the arrays are left unspecified.
 *
 * The mask is static for given (frames, tokens_per_frame, w0). Build it once, copy it to
 * the device, and reuse it for every batch, head and call.
 */
int32_t radial_build_mask(int32_t frames, int32_t tokens_per_frame, int32_t w0, int32_t block,
                          int32_t* row_ptr, int32_t* col_idx, int64_t nnz_capacity);

/*
 * radial_mask_dims_grid, radial_build_mask_grid — the same two calls for the 2-D grid
 * variant of the rule (the radial-attention-video SKILL.md page, Step 1, its grid-distance
 * helper): each frame is a latent grid of grid_h rows of grid_w columns stored row by row
 * (tokens_per_frame = grid_h * grid_w; in-frame index s sits at row s / grid_w, column
 * s % grid_w), and the spatial distance is the Manhattan distance between grid positions:
 *
 *   key allowed <=> (|y_q - y_k| + |x_q - x_k|) * 2^floor(log2(|f_q - f_k| + 1)) < W0.
 *
 * grid_h = 1 gives the 1-D masks of radial_mask_dims / radial_build_mask. Arguments,
 * outputs and errors are as there, with grid_h and grid_w in place of tokens_per_frame:
 * INVALID_ARG if frames, grid_h, grid_w or w0 is <= 0; TOO_LARGE if
 * frames * grid_h * grid_w or the active-block count does not fit in int32.
 */
int32_t radial_mask_dims_grid(int32_t frames, int32_t grid_h, int32_t grid_w, int32_t w0,
                              int32_t block, int32_t* nb_out, int64_t* nnz_out);
int32_t radial_build_mask_grid(int32_t frames, int32_t grid_h, int32_t grid_w, int32_t w0,
                               int32_t block, int32_t* row_ptr, int32_t* col_idx,
                               int64_t nnz_capacity);

/*
 * radial_build_pairs — choose the pairs of query-block rows that the forward kernel
 * computes together. Host code, deterministic.
 *
 * The kernel gives each workgroup two rows and walks the union of their key-block
 * lists: a tile in both rows is copied once for both, a tile in only one leaves the
 * other row's waves idle for that step. The pairing changes no result (each row's
 * output depends only on its own key blocks), only the time. This builder scores
 * candidate partners at row offsets 1, 2, 3 and, when tokens_per_frame > 0, about one
 * and two frames (round(k * tokens_per_frame / 128) + {-1, 0, 1}, k = 1, 2) by the
 * number of key blocks they share, and matches greedily, best score first. It follows
 * "Radial Attention: A Breakthrough in Efficient Long Video Generation", How Radial
 * Attention Works: the window narrows with frame distance, so rows at the same
 * spatial position in neighbouring frames share most of their distant-frame blocks.
 *
 * nb, row_ptr, col_idx: a block mask in host memory (radial_build_mask's output, or any
 *            mask with ascending rows; unsorted rows still give a valid pairing).
 * tokens_per_frame: the frame length of the video, or 0 for no frame structure.
 * pairs:     caller-owned host array of at least 2 * nb int32. On return, entries 2i and
 *            2i + 1 (i < *npairs_out) hold the rows (a, b) of pair i with a < b, or
 *            (a, -1) for a row that runs alone. Every row of [0, nb) appears exactly
 *            once. The pairs come in the order the kernel should take them: by the
 *            length of their union (the number of distinct key blocks of the two rows)
 *            in bands of 16 blocks, longest band first, and by a within a band. Each
 *            XCD takes a head's pairs in contiguous runs of the table (the whole table,
 *            or one of 2, 4 or 8 runs when XCDs share a head), so the pairs it runs at
 *            once have nearly equal length and lie close in the sequence: their
 *            workgroups walk their lists in step and share K/V tiles in that XCD's L2.
 * npairs_out: receives the pair count, between ceil(nb / 2) and nb (ceil(nb / 2) unless
 *            rows are left alone).
 * Cost: about 18 * nnz merge steps. Above 2^28 steps (dense masks of many thousand
 * blocks) it returns the adjacent pairing (2p, 2p + 1) instead.
 *
 * Errors: INVALID_ARG (null pointer, nb <= 0, tokens_per_frame < 0, row_ptr not starting
 * at 0 or decreasing).
 */
int32_t radial_build_pairs(int32_t nb, const int32_t* row_ptr, const int32_t* col_idx,
                           int32_t tokens_per_frame, int32_t* pairs, int32_t* npairs_out);

/*
 * radial_attn_fwd — block-sparse softmax attention forward pass on the GPU. The call is
 * asynchronous on `stream`.
 *
 * q, k, v, o: device pointers to bf16 tensors of logical shape [batch, heads, seqlen,
 *             head_dim]. Element (b, h, t, d) is at b*stride_b + h*stride_h +
 *             t*stride_s + d, with strides counted in elements and shared by all four
 *             tensors. The head_dim axis must be contiguous. [B,H,n,D] and [B,n,H,D]
 *             both work without a copy. o is written for rows t < seqlen only.
 * lse:        optional device pointer (may be null) to float32 [batch, heads, seqlen],
 *             contiguous. It receives the natural-log log-sum-exp of each row's scaled
 *             scores over that row's key set.
 * row_ptr, col_idx: the block mask from radial_build_mask, copied to device memory.
 *             nb = ceil(seqlen / 128). Column indices outside [0, nb) are skipped.
 *             Every row must have at least one active block, which is always true of a
 *             radial mask (the diagonal is allowed).
 * pairs, npairs: optional device copy of radial_build_pairs' output (npairs pairs of
 *             two int32). Null computes the adjacent pairs (2p, 2p + 1) and ignores
 *             npairs. A table must list every row once; entries outside [0, nb) are
 *             treated as absent rows (never read or written), and a row listed twice is
 *             computed twice.
 * scale:      softmax scale, finite and >= 0 (head_dim^-0.5 is the usual value).
 * element_tokens_per_frame, element_w0, element_grid_w: 0 for block semantics
 *             (every real key of an active block takes part; the other two are then
 *             ignored). A frame length of 128 .. 2^22 and W0 >= 1 switch on element
 *             masking: inside the active blocks, key j takes part for query i
 *             only if |s_i - s_j| * 2^floor(log2(|f_i - f_j| + 1)) < W0, with
 *             f = t / frame length and s = t % frame length (frame-major tokens), the
 *             rule of "Radial Attention: A Breakthrough in Efficient Long Video
 *             Generation", How Radial Attention Works, applied entry by entry, masked
 *             scores being -inf before the softmax (the radial-attention-video SKILL.md
 *             page, Step 1). Pass the mask's own frame length and W0; a key the rule
 *             allows outside the CSR's blocks is not visited. Every row must keep at
 *             least one allowed key (the diagonal always is when the CSR comes from
 *             radial_build_mask with the same frame length and W0); a row with none
 *             gets NaN. element_grid_w = 0 takes that 1-D distance |s_i - s_j|; a
 *             divisor W of the frame length takes the grid distance of
 *             radial_build_mask_grid instead (frames of frame length / W rows of W
 *             tokens, |y_i - y_j| + |x_i - x_j| with y = s / W, x = s % W).
 * stream:     a hipStream_t, or null for the default stream.
 *
 * Keys at or past seqlen in the last block are excluded. Rows at or past seqlen are
 * never read or written. Accumulation is fp32, and probabilities are rounded to bf16
 * before the P*V product (the row sum adds them unrounded). Buffers must stay alive and
 * unmodified until the stream work has finished.
 *
 * Scheduling state. The kernel runs one workgroup per compute unit; the workgroups take
 * (batch, head, query-block pair) items from atomic counters. The counters live in a
 * ring of 256 slots in the library's static device memory (one copy per device, zero
 * when the library loads); each launch uses one slot and its kernel leaves that slot at
 * zero when it ends. Results do not depend on which workgroup computes which item.
 *  - Eager calls rotate through slots 0..127 of the current device. Each slot keeps an
 *    event recorded after its last launch; when a call finds that launch unfinished,
 *    it makes `stream` wait for it first (hipStreamWaitEvent), so two kernels never use
 *    one slot at the same time, whatever the number of calls in flight and of streams.
 *    The choice of a slot and its event are guarded by a lock: calls from several host
 *    threads are safe. The events are created on first use and live until the process
 *    ends.
 *  - A call made while `stream` is being captured into a graph takes its slot from
 *    128..255 in turn and records no event (a graph cannot wait for an event recorded
 *    outside it). A graph's slot is never an eager call's. Unchecked: two replays of
 *    graphs whose captures took the same slot (captures 128 apart), running at the
 *    same time on different streams, would split each other's items; the replays of one
 *    graph are ordered by HIP.
 *
 * Errors: INVALID_ARG (null pointer, size <= 0, bad scale, stride_s < head_dim, a pair
 * table with npairs outside [ceil(nb / 2), nb], element masking with a frame length
 * other than 0 below 128 or above 2^22, with W0 < 1, or with a grid width that is
 * negative or does not divide the frame length),
 * UNSUPPORTED_HEAD_DIM, SHAPE_MISMATCH, MISALIGNED (q/k/v/o not 16-byte aligned, or a
 * stride not a multiple of 8 elements), TOO_LARGE (batch*heads*pairs work items
 * above 2^31 - 1, nb above 16352, or a 128-row tile past 2^31 bytes), HIP (the device
 * query, the capture query or the launch failed).
 */
int32_t radial_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int32_t* row_ptr, const int32_t* col_idx, int32_t nb,
                        const int32_t* pairs, int32_t npairs, float scale,
                        int32_t element_tokens_per_frame, int32_t element_w0,
                        int32_t element_grid_w, int32_t batch,
                        int32_t heads, int32_t seqlen, int32_t head_dim, int64_t stride_b,
                        int64_t stride_h, int64_t stride_s, void* stream);

/*
 * radial_element_table_bytes — size of the element table of a mask with nnz active
 * blocks: 2048 bytes per block (its 128 x 128 element decisions, one bit each).
 *
 * nnz:    the CSR's number of active blocks (row_ptr[nb]), >= 0.
 * bytes:  out (host): nnz * 2048.
 *
 * Errors: INVALID_ARG (null bytes, nnz < 0), TOO_LARGE (nnz above 2^31 - 1).
 */
int32_t radial_element_table_bytes(int64_t nnz, int64_t* bytes);

/*
 * radial_build_element_table — stores the element rule's decisions for every active block
 * of a CSR, once per mask, so that radial_attn_fwd_element_table reads them instead of
 * evaluating the rule on every tile it visits. The call is asynchronous on `stream` (one
 * small kernel; the mask is static, "Radial Attention: A Breakthrough in Efficient Long
 * Video Generation", How Radial Attention Works).
 *
 * The decisions are those of radial_attn_fwd's element masking with the same
 * element_tokens_per_frame, element_w0 and element_grid_w (the rule of that page applied
 * to single entries, with frame-major coordinates as on the radial-attention-video
 * SKILL.md page, Step 1), taken by the same device code, so the forward from the table
 * equals the forward with those arguments bit for bit.
 *
 * row_ptr, col_idx:  the block mask (device, int32, nb + 1 and nnz entries), each row's
 *                    columns strictly ascending within [0, nb), as radial_build_mask and
 *                    radial_build_mask_grid give. A column outside [0, nb) gets no bits.
 * nb, nnz:           blocks per side and active blocks (row_ptr[nb], known to the host).
 * element_tokens_per_frame, element_w0, element_grid_w: as for radial_attn_fwd's element
 *                    masking; the frame length must be set (128 .. 2^22).
 * table:             device, caller-owned, 16-byte aligned, at least table_bytes >=
 *                    radial_element_table_bytes(nnz) bytes. Entry j (2048 bytes) belongs to
 *                    CSR entry j: for the query wave w (queries 32w .. 32w + 31 of the
 *                    block's row) and lane l, the 8 bytes at 512w + 8l hold bit 16g + e =
 *                    whether query 32w + l % 32 meets key 32g + 8(e / 4) + 4(l / 32) + e % 4
 *                    of the block (g < 4, e < 16; block-relative indices).
 * stream:            a hipStream_t, or null for the default stream.
 *
 * Errors: INVALID_ARG (null pointer, nb <= 0, nnz < 0, element arguments radial_attn_fwd
 * would refuse, or a zero frame length), TOO_LARGE (nb above 16352, nnz above 2^31 - 1),
 * CAPACITY (table_bytes too small), MISALIGNED (table), HIP (the launch failed).
 */
int32_t radial_build_element_table(const int32_t* row_ptr, const int32_t* col_idx, int32_t nb,
                                   int64_t nnz, int32_t element_tokens_per_frame,
                                   int32_t element_w0, int32_t element_grid_w, void* table,
                                   int64_t table_bytes, void* stream);

/*
 * radial_attn_fwd_element_table — radial_attn_fwd with element masking from an element
 * table (radial_build_element_table on the same row_ptr and col_idx) instead of the
 * element arguments. Every other argument, the scheduling state and the errors are
 * radial_attn_fwd's; element_table (device) must be non-null and 16-byte aligned
 * (INVALID_ARG, MISALIGNED). The output and lse equal radial_attn_fwd's with the
 * table's element arguments bit for bit. The kernel takes the table entry of each
 * active block by its position in the block's CSR row, so the CSR must be the one the
 * table was built from, rows strictly ascending within [0, nb); for any other CSR the
 * masking is unspecified (reads stay within the row's entries).
 */
int32_t radial_attn_fwd_element_table(const void* q, const void* k, const void* v, void* o,
                                      float* lse, const int32_t* row_ptr,
                                      const int32_t* col_idx, int32_t nb, const int32_t* pairs,
                                      int32_t npairs, float scale, const void* element_table,
                                      int32_t batch, int32_t heads, int32_t seqlen,
                                      int32_t head_dim, int64_t stride_b, int64_t stride_h,
                                      int64_t stride_s, void* stream);

/*
 * radial_attn_fwd_rule — radial_attn_fwd with the block mask derived on the fly in the
 * kernel instead of read from a CSR. The call is asynchronous on `stream`.
 *
 * Each workgroup marks its two query-block rows' active key blocks itself, from the
 * same rule and with the same sweep as radial_build_mask (grid_w = 0) or
 * radial_build_mask_grid (grid_w > 0): the mask is static and determined by (frames,
 * tokens_per_frame, grid_w, w0) ("Radial Attention: A Breakthrough in Efficient Long
 * Video Generation", How Radial Attention Works), so it need not be stored. Rows are
 * visited in the same ascending key-block order as with the built CSR, so the output
 * and lse equal radial_attn_fwd's on that CSR bit for bit.
 *
 * frames, tokens_per_frame, w0: the video and base window; seqlen = frames *
 *             tokens_per_frame (at most 16352 * 128 tokens).
 * grid_w:     0 for the 1-D spatial distance, or the grid width (a divisor of
 *             tokens_per_frame) for the 2-D grid distance.
 * element:    nonzero applies the same rule to single entries inside the active blocks
 *             (radial_attn_fwd's element masking with element_tokens_per_frame =
 *             tokens_per_frame, element_w0 = w0, element_grid_w = grid_w).
 * q, k, v, o, lse, pairs, npairs, scale, batch, heads, head_dim, strides, stream: as
 *             radial_attn_fwd (a pair table, if given, comes from radial_build_pairs on
 *             the built mask; null pairs rows 2p and 2p + 1).
 *
 * Errors: INVALID_ARG (frames, tokens_per_frame or w0 <= 0, a grid width that is
 * negative or does not divide tokens_per_frame, element masking with a frame outside
 * 128 .. 2^22, and radial_attn_fwd's other argument errors), UNSUPPORTED_HEAD_DIM,
 * MISALIGNED, TOO_LARGE (a sequence above 16352 * 128 tokens, work items past int32, or
 * more than 2^16 marking steps per row: (frame pieces of a 128-token block) x frames x
 * grid rows, a few thousand for real videos), HIP.
 */
int32_t radial_attn_fwd_rule(const void* q, const void* k, const void* v, void* o, float* lse,
                             int32_t frames, int32_t tokens_per_frame, int32_t grid_w,
                             int32_t w0, int32_t element, const int32_t* pairs,
                             int32_t npairs, float scale, int32_t batch, int32_t heads,
                             int32_t head_dim, int64_t stride_b, int64_t stride_h,
                             int64_t stride_s, void* stream);

/*
 * radial_attn_fwd_varlen — radial_attn_fwd over a batch of videos of different lengths
 * (each sample its own frame count, so its own mask), packed into one sequence. The
 * call is asynchronous on `stream`.
 *
 * q, k, v, o: device bf16 [total_tokens, heads, head_dim] (any layout with element
 *             strides stride_s between tokens and stride_h between heads, shared by all
 *             four, head_dim contiguous). Sample b holds tokens [t_b, t_b + seq_tokens[b])
 *             with t_b the sum of the lengths before it.
 * lse:        optional device fp32 [heads, total_tokens], contiguous.
 * seq_tokens: host array of batch lengths (each >= 1); 1 <= batch <= 64.
 * row_ptr, col_idx: the samples' block masks (device), concatenated: sample b's nb_b + 1
 *             row_ptr entries follow those of samples 0 .. b-1 (nb_b = ceil(len / 128)),
 *             and their values index the concatenated col_idx. Column indices count key
 *             blocks within the sample.
 * pairs, npairs: optional pair tables (device, concatenated: sample b's npairs[b] pairs
 *             follow those of the samples before it) and their host array of counts;
 *             null for the adjacent pairs of every sample.
 * Other arguments as radial_attn_fwd; element masking uses each sample's own token
 * indices. The kernel, its work counters and its numerics are radial_attn_fwd's.
 *
 * Errors: INVALID_ARG (null pointer, batch <= 0, a length <= 0, pairs without npairs, a
 * pair count outside [ceil(nb_b / 2), nb_b], heads <= 0, stride_s < head_dim, bad scale
 * or element arguments), UNSUPPORTED_HEAD_DIM, MISALIGNED, TOO_LARGE (batch above 64,
 * a sample above 16352 blocks, totals past int32), HIP.
 */
int32_t radial_attn_fwd_varlen(const void* q, const void* k, const void* v, void* o,
                               float* lse, const int32_t* seq_tokens, int32_t batch,
                               const int32_t* row_ptr, const int32_t* col_idx,
                               const int32_t* pairs, const int32_t* npairs, float scale,
                               int32_t element_tokens_per_frame, int32_t element_w0,
                               int32_t element_grid_w,
                               int32_t heads, int32_t head_dim, int64_t stride_h,
                               int64_t stride_s, void* stream);

/*
 * radial_attn_fwd_varlen_element_table — radial_attn_fwd_varlen with element masking from
 * an element table instead of the element arguments: the samples' tables
 * (radial_build_element_table on each sample's own mask) concatenated in sample order, so
 * that entry j belongs to entry j of the concatenated col_idx. Every other argument and
 * error is radial_attn_fwd_varlen's; element_table (device) must be non-null and 16-byte
 * aligned (INVALID_ARG, MISALIGNED). The output and lse equal radial_attn_fwd_varlen's
 * with the tables' element arguments bit for bit; the CSR rows must be strictly
 * ascending within each sample's [0, nb), as radial_attn_fwd_element_table requires.
 */
int32_t radial_attn_fwd_varlen_element_table(const void* q, const void* k, const void* v,
                                             void* o, float* lse, const int32_t* seq_tokens,
                                             int32_t batch, const int32_t* row_ptr,
                                             const int32_t* col_idx, const int32_t* pairs,
                                             const int32_t* npairs, float scale,
                                             const void* element_table, int32_t heads,
                                             int32_t head_dim, int64_t stride_h,
                                             int64_t stride_s, void* stream);

/*
 * radial_attn_fwd_varlen_rule — radial_attn_fwd_varlen with each sample's block mask
 * derived on the fly in the kernel (as radial_attn_fwd_rule does) instead of read from a
 * CSR. The call is asynchronous on `stream`.
 *
 * frames:     host array of batch frame counts (each >= 1); sample b holds
 *             frames[b] * tokens_per_frame tokens; 1 <= batch <= 64.
 * tokens_per_frame, grid_w, w0, element: the rule, as for radial_attn_fwd_rule.
 * pairs, npairs: optional pair tables as for radial_attn_fwd_varlen.
 * Other arguments as radial_attn_fwd_varlen. Output and lse equal radial_attn_fwd_varlen's
 * on the samples' built masks bit for bit.
 *
 * Errors: as radial_attn_fwd_varlen and radial_attn_fwd_rule (a frame count <= 0 is
 * INVALID_ARG; a sample past 16352 blocks or 2^16 marking steps per row is TOO_LARGE).
 */
int32_t radial_attn_fwd_varlen_rule(const void* q, const void* k, const void* v, void* o,
                                    float* lse, const int32_t* frames, int32_t batch,
                                    int32_t tokens_per_frame, int32_t grid_w, int32_t w0,
                                    int32_t element, const int32_t* pairs,
                                    const int32_t* npairs, float scale, int32_t heads,
                                    int32_t head_dim, int64_t stride_h, int64_t stride_s,
                                    void* stream);

/*
 * radial_transpose_mask — the transposed block mask, for the backward pass: for key
 * block c, the query blocks whose rows list it, in ascending order. Host code.
 *
 * nb, row_ptr, col_idx: a block mask in host memory. Entries outside [0, nb) are dropped.
 * col_ptr:   caller-owned host array of nb + 1 int32; col_ptr[0] = 0 and column c's query
 *            blocks are row_idx[col_ptr[c] .. col_ptr[c+1]).
 * row_idx:   caller-owned host array of at least row_ptr[nb] int32.
 * A radial mask is symmetric at block level, so its transpose equals itself; other
 * masks need this call.
 *
 * Errors: INVALID_ARG (null pointer, nb <= 0, row_ptr not starting at 0 or decreasing).
 */
int32_t radial_transpose_mask(int32_t nb, const int32_t* row_ptr, const int32_t* col_idx,
                              int32_t* col_ptr, int32_t* row_idx);

/*
 * radial_attn_bwd — gradients of radial_attn_fwd: dq, dk, dv for the output gradient
 * dout. The pages fine-tune through the attention with LoRA (the radial-attention-video
 * SKILL.md page, Step 4: loss.backward() through the attention layers). With P the
 * forward's softmax over each row's key set and D_i = <dout_i, o_i>:
 *     dv_j = sum_i P_ij dout_i,  dS_ij = P_ij (<dout_i, v_j> - D_i),
 *     dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i.
 * P is recomputed from the forward's lse: P_ij = exp(scale <q_i, k_j> - lse_i). The call
 * is asynchronous on `stream` and runs three kernels (D, then dq, then dk and dv).
 *
 * q, k, v, o, dout, dq, dk, dv: device bf16 [batch, heads, seqlen, head_dim] sharing one
 *             set of element strides (as in radial_attn_fwd); o is the forward's output
 *             for these q, k, v and mask. dq, dk, dv are written for rows < seqlen.
 * lse:        the forward's lse output (fp32 [batch, heads, seqlen], contiguous).
 * delta:      caller-owned device workspace of 2 * batch * heads * seqlen fp32: the
 *             call writes D_i into the first half and lse_i log2(e) into the second,
 *             both [batch, heads, seqlen], and reads them back in its later kernels.
 * row_ptr, col_idx: the block mask used by the forward (device).
 * col_ptr, row_idx: its transpose from radial_transpose_mask (device). For a radial mask
 *             these may be row_ptr and col_idx themselves.
 * scale, element_tokens_per_frame, element_w0, element_grid_w: as passed to the forward.
 * Accumulation is fp32; P and dS enter the matrix products as bf16.
 *
 * Errors: as radial_attn_fwd (INVALID_ARG, UNSUPPORTED_HEAD_DIM, SHAPE_MISMATCH,
 * MISALIGNED: also lse or delta not 4-byte aligned, TOO_LARGE: batch*heads*nb work items
 * or batch*heads*seqlen rows above 2^31 - 1, HIP).
 */
int32_t radial_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        float* delta, const int32_t* row_ptr, const int32_t* col_idx,
                        const int32_t* col_ptr, const int32_t* row_idx, int32_t nb,
                        float scale, int32_t element_tokens_per_frame, int32_t element_w0,
                        int32_t element_grid_w,
                        int32_t batch, int32_t heads, int32_t seqlen, int32_t head_dim,
                        int64_t stride_b, int64_t stride_h, int64_t stride_s, void* stream);

/*
 * radial_attn_bwd_element_table — radial_attn_bwd with element masking from an element
 * table (radial_build_element_table on the same row_ptr and col_idx) instead of the
 * element arguments. Every other argument, the workspace and the errors are
 * radial_attn_bwd's; element_table (device) must be non-null and 16-byte aligned
 * (INVALID_ARG, MISALIGNED). The gradients equal radial_attn_bwd's with the table's
 * element arguments bit for bit.
 *
 * The dq kernel takes the decisions of row block i's t-th active block from table entry
 * row_ptr[i] + t. The dK/dV kernel walks key block j's column (col_ptr, row_idx) and,
 * since the rule is symmetric, takes the decisions of its t-th entry from row j's t-th
 * entry row_ptr[j] + t: the mask must be symmetric (its transpose equal to itself, as
 * every radial mask is). For any other mask dK and dV use unspecified decisions (entries
 * past row j's end read as all masked; reads stay within the table).
 */
int32_t radial_attn_bwd_element_table(const void* q, const void* k, const void* v,
                                      const void* o, const void* dout, const float* lse,
                                      void* dq, void* dk, void* dv, float* delta,
                                      const int32_t* row_ptr, const int32_t* col_idx,
                                      const int32_t* col_ptr, const int32_t* row_idx,
                                      int32_t nb, float scale, const void* element_table,
                                      int32_t batch, int32_t heads, int32_t seqlen,
                                      int32_t head_dim, int64_t stride_b, int64_t stride_h,
                                      int64_t stride_s, void* stream);

/*
 * radial_attn_bwd_noalloc — radial_attn_bwd without the delta workspace argument, for
 * callers that cannot allocate device memory: code under graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. The call allocates nothing: its workspace (D_i
 * and the base-2 lse, two fp32 per row) is a static device array of the library,
 * 2 * 2^23 fp32 values (64 MiB) on each device the library runs on, held until the
 * process ends.
 *
 * Arguments, results and numerics are radial_attn_bwd's (the same kernels), without
 * `delta`. The workspace keeps the last call's values; nothing needs to start at zero.
 * Every call on one device shares that device's workspace, so two calls that overlap
 * on one device (on different streams, or graph replays running at once) race and give
 * wrong gradients; calls on one stream are ordered and safe.
 *
 * Errors: as radial_attn_bwd, plus TOO_LARGE when batch * heads * seqlen exceeds 2^23
 * (the rows the workspace holds), checked before any HIP call; HIP also when the workspace's device
 * address cannot be looked up.
 */
int32_t radial_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                                const void* dout, const float* lse, void* dq, void* dk,
                                void* dv, const int32_t* row_ptr, const int32_t* col_idx,
                                const int32_t* col_ptr, const int32_t* row_idx, int32_t nb,
                                float scale, int32_t element_tokens_per_frame,
                                int32_t element_w0, int32_t element_grid_w, int32_t batch,
                                int32_t heads, int32_t seqlen, int32_t head_dim,
                                int64_t stride_b, int64_t stride_h, int64_t stride_s,
                                void* stream);

/*
 * radial_attn_bwd_varlen — radial_attn_bwd over a packed varlen batch (the backward of
 * radial_attn_fwd_varlen). The call is asynchronous on `stream`.
 *
 * q, k, v, o, dout, dq, dk, dv: device bf16 [total_tokens, heads, head_dim] with element
 *             strides stride_s between tokens and stride_h between heads, shared by all
 *             eight, head_dim contiguous; sample b holds the next seq_tokens[b] tokens.
 * lse:        the forward's fp32 [heads, total_tokens] output (contiguous).
 * delta:      caller-owned fp32 workspace of 2 * heads * total_tokens (D_i, then
 *             lse_i log2(e), each [heads, total_tokens]).
 * seq_tokens: host array of batch lengths (each >= 1); 1 <= batch <= 64.
 * row_ptr, col_idx, col_ptr, row_idx: the samples' block masks and their transposes
 *             (device), each concatenated as radial_attn_fwd_varlen takes row_ptr and
 *             col_idx: sample b's nb_b + 1 pointer entries follow those of the samples
 *             before it and index the concatenated index array; indices count blocks
 *             within the sample.
 * scale, element arguments: as passed to the forward.
 * Each sample's gradients equal radial_attn_bwd's on that sample alone (the same kernels
 * on the same tiles).
 *
 * Errors: INVALID_ARG (null pointer, batch <= 0, a length <= 0, heads <= 0, bad scale or
 * element arguments, stride_s < head_dim), UNSUPPORTED_HEAD_DIM, MISALIGNED, TOO_LARGE
 * (batch above 64, totals past int32), HIP.
 */
int32_t radial_attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                               const void* dout, const float* lse, void* dq, void* dk,
                               void* dv, float* delta, const int32_t* seq_tokens,
                               int32_t batch, const int32_t* row_ptr, const int32_t* col_idx,
                               const int32_t* col_ptr, const int32_t* row_idx, float scale,
                               int32_t element_tokens_per_frame, int32_t element_w0,
                               int32_t element_grid_w, int32_t heads, int32_t head_dim,
                               int64_t stride_h, int64_t stride_s, void* stream);

/*
 * radial_attn_bwd_varlen_element_table — radial_attn_bwd_varlen with element masking from
 * the concatenated element table of radial_attn_fwd_varlen_element_table. Every other
 * argument and error is radial_attn_bwd_varlen's; element_table must be non-null and
 * 16-byte aligned. Gradients equal radial_attn_bwd_varlen's bit for bit. As for
 * radial_attn_bwd_element_table, every sample's mask must be symmetric (radial masks
 * are); otherwise dK and dV use unspecified decisions, with reads inside the table.
 */
int32_t radial_attn_bwd_varlen_element_table(const void* q, const void* k, const void* v,
                                             const void* o, const void* dout,
                                             const float* lse, void* dq, void* dk, void* dv,
                                             float* delta, const int32_t* seq_tokens,
                                             int32_t batch, const int32_t* row_ptr,
                                             const int32_t* col_idx, const int32_t* col_ptr,
                                             const int32_t* row_idx, float scale,
                                             const void* element_table, int32_t heads,
                                             int32_t head_dim, int64_t stride_h,
                                             int64_t stride_s, void* stream);

/* radial_error_string — a static, human-readable text for a return code. */
const char* radial_error_string(int32_t code);

#ifdef __cplusplus
}
#endif

#endif /* RADIAL_ATTN_H */
