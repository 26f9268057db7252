/*
 * sta.h - C ABI of the Sliding Tile Attention (STA) forward library (gfx950).
 *
 * The operation is the one described by the "Sliding Tile Atteniton Kernel"
 * README (FastVideo, sta_kernel/thunderkitten), sections "Usage" and "Why is
 * STA Fast?": softmax attention over a T x H x W video latent cut into tiles
 * of (6, 8, 8) tokens, where each query tile attends to a per-head window of
 * whole key tiles (given in tiles), plus an optional segment of 256 padded
 * text slots of which the first `text_length` are valid. The attention map
 * holds only fully-dense or fully-empty tile blocks.
 *
 * Video sizes need not be tile multiples. The page's kernel takes only
 * multiples of (6, 8, 8) and leaves other sizes to the caller; this library
 * reads them as follows: the tile grid is (n_t, n_h, n_w) = (ceil(T/6),
 * ceil(H/8), ceil(W/8)), the last tile along an axis holds the remainder
 * (the tokens of tile (i, j, k) are those of its 6x8x8 box that exist),
 * windows are placed on that grid exactly as for multiples, and a query sees
 * the tokens that exist in its window's tiles. For multiples this is the
 * page's operation unchanged.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Sequence order ("raster"): video token (t, h, w) is row (t*H + h)*W + w;
 *   when has_text != 0 the 256 text slots follow as rows [T*H*W, T*H*W+256).
 *   S = T*H*W + (has_text ? 256 : 0).
 * - Tensors q, k, v, out are bf16, row-major [batch][heads][S][head_dim].
 *   lse is fp32 [batch][heads][S].
 * - Device pointers are HIP device (or managed) memory, 16-byte aligned.
 *   The caller owns every buffer and the library allocates no device
 *   memory. Its only state is a per-device cache, filled on the first call
 *   on a device, of how many workgroups of each persistent kernel fit on
 *   that device at once (a value the runtime reports and that never
 *   changes); it affects no result. Calls on different buffers may run
 *   concurrently.
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   Work is enqueued asynchronously; the return value reports argument
 *   errors (found on the host before anything is enqueued) and launch
 *   errors. Faults inside kernels surface at the caller's next stream sync.
 * - Environment: with STA_LOG set to anything but "" or "0", every
 *   sta_forward and sta_backward call (and their _timed and _noalloc forms)
 *   prints one line to stderr, after its arguments are validated and before
 *   it enqueues anything: the geometry, the query units per head and their
 *   kind (single tiles, 2x2 squares, Hilbert runs), the text parts, head 0's
 *   window and the workspace bytes.
 * - window_sizes is a HOST array of heads*3 int32: (w_t, w_h, w_w) in tiles
 *   for head 0, then head 1, ... Each component must lie in [1, n_axis]
 *   where (n_t, n_h, n_w) = (ceil(T/6), ceil(H/8), ceil(W/8)). At the grid
 *   border the window is shifted inward (start = clamp(c - w/2, 0, n - w)
 *   per axis) so every video query sees exactly w_t*w_h*w_w tiles.
 */
#ifndef STA_H
#define STA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  STA_OK = 0,
  STA_ERR_NULL = 1,      /* a required pointer is NULL, or batch/heads <= 0      */
  STA_ERR_SHAPE = 2,     /* T,H,W not positive; head_dim not 64 or 128;
                            heads > STA_MAX_HEADS; a tile-grid axis > 1023
                            tiles; or sizes too large to index                 */
  STA_ERR_WINDOW = 3,    /* a window component outside [1, n_axis]              */
  STA_ERR_TEXT = 4,      /* text_length outside [0, 256], or != 0 without text  */
  STA_ERR_ALIGN = 5,     /* a device pointer is not 16-byte aligned             */
  STA_ERR_WORKSPACE = 6, /* workspace NULL or smaller than sta_workspace_bytes  */
  STA_ERR_HIP = 7,       /* the HIP runtime reported an error at launch         */
  STA_ERR_ALIAS = 8,     /* out (or lse) overlaps an input                      */
  STA_ERR_SCRATCH = 9    /* sta_forward_noalloc: the shape needs more workspace
                            than its fixed scratch (STA_NOALLOC_SCRATCH_BYTES)  */
} sta_status;

#define STA_MAX_HEADS 256
#define STA_TEXT_SLOTS 256

typedef struct {
  int32_t batch;    /* B >= 1                                  */
  int32_t heads;    /* 1 .. STA_MAX_HEADS                      */
  int32_t head_dim; /* D: 64 or 128                            */
  int32_t T, H, W;  /* video size in tokens, each >= 1             */
} sta_dims;

/* Human-readable name of a status code (static string, never NULL). */
const char* sta_status_str(sta_status s);

/* Sequence length S for these dims (0 if dims are invalid). */
int64_t sta_seq_len(const sta_dims* dims, int32_t has_text);

/*
 * Rows per (batch, head) of the tile-major order (0 if dims are invalid):
 * n_t*n_h*n_w*384 (+256 with text). Equal to S for video sizes that are tile
 * multiples; otherwise it includes the padding rows of partial tiles.
 */
int64_t sta_tiled_seq_len(const sta_dims* dims, int32_t has_text);

/*
 * Bytes of device workspace sta_forward needs for these arguments, or 0 if
 * the arguments are invalid. Depends on the windows (they decide the query
 * units, see sta_forward). Pure host arithmetic: no HIP call.
 */
size_t sta_workspace_bytes(const sta_dims* dims, const int32_t* window_sizes,
                           int32_t has_text);

/*
 * STA forward: out = softmax(q k^T / sqrt(D), masked to the sliding tile
 * window and the valid text keys) v, and lse = natural log of the softmax
 * denominator, per query row.
 *
 * Which keys a query row sees (README "Usage": window in tiles, text length,
 * Hunyuan-style text mode or StepVideo-style has_text = 0):
 *   video query -> video keys of the w_t x w_h x w_w key tiles of its
 *                  clamped window, and text keys [0, text_length);
 *   text query (every one of the 256 slots, padded slots included)
 *                -> all video keys and text keys [0, text_length).
 * Text K/V rows at or after text_length never influence any result (their
 * contents, even non-finite values, are ignored).
 *
 * q, k, v   : device, bf16 [B][heads][S][D], raster order, read only.
 * out       : device, bf16 [B][heads][S][D], written; must not overlap inputs.
 * lse       : device, fp32 [B][heads][S], written; may be NULL to skip it.
 * workspace : device, >= sta_workspace_bytes(dims, window_sizes, has_text)
 *             bytes, 256-byte aligned; contents on entry are ignored and on
 *             return are unspecified. Calls that share a workspace must be
 *             ordered on one stream.
 * Returns STA_OK once the two launches (the work order of query units, and
 * the fused attention kernel, which reads q, k and v and writes out/lse in
 * raster order, all through the tile map, and enumerates each unit's window
 * of key tiles itself) are enqueued on `stream`. The workspace holds the work
 * order (4 bytes per query unit: B*heads*(n_t*n_h*n_w + has_text) units), 2 KB
 * of work-queue heads and a 256-byte zero row: a few KB to a few hundred KB.
 * One-frame videos (T = 1, the 2D-image reading of README "How Does STA
 * Work?"; every tile is one frame of at most 8x8 tokens): when
 * every head's window spans at least 2 tiles along each axis that has at
 * least 2 tiles, a query unit is a 2x2 square of tiles (B*heads*
 * ceil(n_h/2)*ceil(n_w/2) video units), and with text on images of 256 tiles
 * or more the text rows are split over P = min(8, tiles/128) units by key
 * tiles, whose fp32 partial results (B*heads*P*256*(D+2)*4 bytes of
 * workspace) a third launch merges. The results are the same function of
 * the inputs either way.
 * The attention launch is a persistent grid (one workgroup per resident slot
 * on the current device) whose workgroups take query units from per-XCD
 * queues, their own XCD's first; which workgroup runs which unit varies from
 * call to call, the results do not.
 */
sta_status sta_forward(const sta_dims* dims, const void* q, const void* k,
                       const void* v, const int32_t* window_sizes,
                       int32_t text_length, int32_t has_text, void* out,
                       float* lse, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * sta_forward with stage timing, for measurement. `events` holds
 * STA_TIMED_EVENTS hipEvent_t handles (as void*, created by the caller);
 * events[0] is recorded on `stream` before the first launch and events[i]
 * after launch i of: 1 work order, 2 fused attention (with, for split text
 * rows, their merge). hipEventElapsedTime
 * between consecutive events then gives each kernel's duration. Nothing else
 * differs from sta_forward; STA_ERR_NULL if events or an entry is NULL.
 */
#define STA_TIMED_EVENTS 3
sta_status sta_forward_timed(const sta_dims* dims, const void* q, const void* k,
                             const void* v, const int32_t* window_sizes,
                             int32_t text_length, int32_t has_text, void* out,
                             float* lse, void* workspace, size_t workspace_bytes,
                             void* stream, void* const* events);

/*
 * sta_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. The
 * arguments and results are those of sta_forward without the workspace; its
 * place is taken by a fixed device array of STA_NOALLOC_SCRATCH_BYTES inside
 * the library, one per GPU, which the GPU holds until the process ends (its
 * address is looked up once per device, on the first call there). Nothing is
 * allocated or freed, by this call or by anything it calls. Every call on a
 * GPU uses that GPU's one array and finds it as the previous call left it;
 * the work-queue heads and the zero row that must start at zero are cleared
 * by the call's own first kernel. Calls that overlap on one GPU (other
 * streams, other threads) race on the array: order them on one stream.
 * Split text rows of one-frame videos are used only when their partial
 * results fit the array; otherwise the text rows stay whole (same results
 * up to rounding order). Returns STA_ERR_SCRATCH, before any launch, when
 * the work order still exceeds STA_NOALLOC_SCRATCH_BYTES (enough for about
 * 260 000 query units, B*heads*(n_t*n_h*n_w + has_text)), STA_ERR_HIP when
 * the array's address cannot be obtained, otherwise what sta_forward
 * returns.
 */
#define STA_NOALLOC_SCRATCH_BYTES (1u << 20)
sta_status sta_forward_noalloc(const sta_dims* dims, const void* q, const void* k,
                               const void* v, const int32_t* window_sizes,
                               int32_t text_length, int32_t has_text, void* out,
                               float* lse, void* stream);

/*
 * Hilbert-window attention on a 2D image ("Boosting 2D Local Attention
 * Efficiency with Hilbert-Guided Sparsity", TLDR and "The Hilbert Curve
 * Advantage": tokens reordered along a Hilbert curve, windows built on that
 * 1D order, run by a block-sparse kernel unchanged). The image is a one-frame
 * video: dims->T = 1 and H = W = 8 * 2^m, so its 8x8 tiles form a 2^m x 2^m
 * grid (n = 4^m tiles); other sizes are STA_ERR_SHAPE. The Hilbert curve of
 * order m on the tile grid runs from tile (0, 0) to tile (2^m - 1, 0) (x =
 * column, y = row); order j visits the quadrants (x low, y low), (x low, y
 * high), (x high, y high), (x high, y low), running the order j - 1 curve
 * transposed, shifted, shifted, and reflected through the anti-diagonal. A
 * 64-token block of the token-level curve is exactly one tile, so the pattern
 * is one of whole tiles. A video query of the tile at curve position i sees
 * the key tiles at positions
 *   STA_HILBERT_SLIDE:  [s, s + W), s = clamp(i - W / 2, 0, n - W)
 *   STA_HILBERT_WINDOW: [W * (i / W), min(W * (i / W) + W, n))
 * with W = window_lens[head] in [1, min(n, 1023)] (else STA_ERR_WINDOW, as is
 * another mode), plus the valid text keys; text queries see every video key
 * and the valid text keys, as in sta_forward. q, k, v, out and lse are laid
 * out as in sta_forward (raster token order; the curve only picks the key
 * tiles, and softmax attention does not depend on the order of the keys).
 * workspace: >= sta_hilbert_workspace_bytes(dims, has_text) bytes, 256-byte
 * aligned, same rules as sta_forward's. With text on images of 256 tiles or
 * more (128 x 128 tokens), it also holds fp32 partial results of the text
 * rows, up to 8 x 256 x (D + 2) floats per (batch, head). Two launches on
 * `stream`, as in sta_forward, and on such images a third, which merges
 * those partial results into the text rows of out and lse; the same argument
 * errors.
 */
#define STA_HILBERT_SLIDE 1
#define STA_HILBERT_WINDOW 2
size_t sta_hilbert_workspace_bytes(const sta_dims* dims, int32_t has_text);
sta_status sta_hilbert_forward(const sta_dims* dims, const void* q, const void* k,
                               const void* v, const int32_t* window_lens, int32_t mode,
                               int32_t text_length, int32_t has_text, void* out,
                               float* lse, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * Raster <-> Hilbert order of the rows of one bf16 tensor [B][heads][S][D] of
 * a 2D image (same shape rules as sta_hilbert_forward; same post): row d of
 * x_hilbert is the token at position d of the order m + 3 curve over the
 * image's tokens (the curve above, at token level), for d < H * W; the 256
 * text rows, when has_text, keep their place. The two buffers must not
 * overlap. sta_hilbert_scatter is the inverse.
 */
sta_status sta_hilbert_gather(const sta_dims* dims, int32_t has_text,
                              const void* x_raster, void* x_hilbert, void* stream);
sta_status sta_hilbert_scatter(const sta_dims* dims, int32_t has_text,
                               const void* x_hilbert, void* x_raster, void* stream);

/*
 * Tile-major gather of one bf16 tensor. The tile is the one the STA README
 * ("Usage") fixes: a cube of (6, 8, 8) video tokens; laying each tile's 384
 * tokens out contiguously turns every dense (query tile, key tile) block of
 * the attention map into a contiguous slab (README "Why is STA Fast?").
 * x_raster [B][heads][S][D] into
 * x_tiled [B][heads][S_t][D] with S_t = sta_tiled_seq_len(dims, has_text).
 * Tile tile = ((t/6)*n_h + h/8)*n_w + w/8 owns the 384 contiguous rows
 * tile*384 ..; its video rows (t, h, w) come first in (frame, row, column)
 * order, i.e. row tile*384 + ((t%6)*ch + h%8)*cw + w%8 where ch and cw are
 * the rows and columns of the tile that exist (8 and 8 except in the last
 * tile along h or w of a size that is not a tile multiple), and the slot's
 * remaining rows (a partial tile's padding) are written as zeros. The text
 * rows follow the video (row n_t*n_h*n_w*384 + slot). For tile multiples
 * S_t = S and this is a plain row permutation. The two buffers must not
 * overlap.
 */
sta_status sta_tile_gather(const sta_dims* dims, int32_t has_text,
                           const void* x_raster, void* x_tiled, void* stream);

/* Inverse of sta_tile_gather (README "Usage": the (6, 8, 8) tile); the padding
 * rows of x_tiled are not read. Same argument rules as sta_tile_gather. */
sta_status sta_tile_scatter(const sta_dims* dims, int32_t has_text,
                            const void* x_tiled, void* x_raster, void* stream);

/*
 * Sizes (in int32 elements) of the three schedule arrays for these
 * arguments: offsets (heads*n_q + 1), key-tile ids and the work order
 * (B*heads*n_q), where n_q = n_t*n_h*n_w query tiles plus one text query
 * unit when has_text. Returns STA_OK or an argument error. Host only.
 */
sta_status sta_schedule_sizes(const sta_dims* dims, const int32_t* window_sizes,
                              int32_t has_text, int64_t* n_offsets,
                              int64_t* n_ids, int64_t* n_work);

/*
 * Build the tile-window schedule on the device.
 *   offsets[hd*n_q + u] .. offsets[hd*n_q + u + 1] delimit, in ids, the key
 *   tiles that query unit u of head hd sees: for a video query tile, the
 *   tiles of its clamped window, ordered by the residues of their tile
 *   coordinates (t mod w_t, h mod w_h, w mod w_w) in nested order with the
 *   last fastest, so query tiles with overlapping windows reach each shared
 *   tile at the same step; for the text unit (u = n_tiles), every tile
 *   0 .. n_tiles-1.
 *   work holds 8 queues of query units ((b*heads + hd)*n_q + u), one per
 *   XCD: queue x is work[x], work[8 + x], work[16 + x], ...; each queue
 *   runs heaviest units first and takes a contiguous run of every class of
 *   equal-cost units.
 * All three arrays are device int32 of the sizes sta_schedule_sizes gives.
 */
sta_status sta_build_schedule(const sta_dims* dims, const int32_t* window_sizes,
                              int32_t text_length, int32_t has_text,
                              int32_t* offsets, int32_t* ids, int32_t* work,
                              void* stream);

/*
 * Bytes of device workspace sta_backward needs for these arguments, or 0 if
 * they are invalid: two fp32 values per row (video rows padded to whole
 * tiles), the forward's tile lists, 4 KB of queue heads and one 256-byte
 * zero row.
 * Pure host arithmetic: no HIP call.
 */
size_t sta_backward_workspace_bytes(const sta_dims* dims, const int32_t* window_sizes,
                                    int32_t has_text);

/*
 * STA backward: the gradients of sta_forward's out with respect to q, k and
 * v, for an upstream gradient dout. With c = 1/sqrt(D), P the probabilities
 * of the forward (softmax over the keys each query row sees, as documented
 * at sta_forward) and delta_i = sum_d dout[i][d] * out[i][d]:
 *   dv_j = sum_i P_ij dout_i,   dS_ij = P_ij (dout_i . v_j - delta_i),
 *   dq_i = c sum_j dS_ij k_j,   dk_j = c sum_i dS_ij q_i.
 * This is the chain rule through the forward's definition (STA README
 * "Usage" and "Why is STA Fast?"; the page shows only the forward call).
 * P is recomputed from q, k and lse; delta from out and dout.
 *
 * q, k, v   : device, bf16 [B][heads][S][D], raster order: the forward's inputs.
 * out, lse  : device, the forward's outputs for these inputs (bf16 rows and
 *             fp32 natural-log lse, as sta_forward writes them). Read only.
 * dout      : device, bf16 [B][heads][S][D], read only. Every row, padded
 *             text query rows included, is a row of the forward's output and
 *             contributes.
 * dq, dk, dv: device, bf16 [B][heads][S][D], written. They must not overlap
 *             each other, an input or the workspace. Text key slots at or
 *             after text_length are seen by no query: their dk and dv rows
 *             are written as zeros. With video sizes that are not tile
 *             multiples, every existing row is written.
 * workspace : device, >= sta_backward_workspace_bytes(...) bytes, 256-byte
 *             aligned; contents on entry ignored, on return unspecified.
 *             Calls that share a workspace must be ordered on one stream.
 * Errors as for sta_forward (all found on the host before any launch).
 * Returns STA_OK once the launches (row statistics, the tile lists, the dq
 * pass, the dk/dv pass) are enqueued on `stream`. The dq and dk/dv launches
 * are persistent grids pulling units from per-XCD queues, like the forward's
 * attention launch.
 */
sta_status sta_backward(const sta_dims* dims, const void* q, const void* k, const void* v,
                        const void* out, const float* lse, const void* dout,
                        const int32_t* window_sizes, int32_t text_length, int32_t has_text,
                        void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * sta_backward with stage timing. `events` holds STA_BWD_TIMED_EVENTS
 * hipEvent_t handles (as void*): events[0] before the first launch, then
 * after 1 row statistics, 2 tile lists, 3 the dq pass, 4 the dk/dv pass.
 * STA_ERR_NULL if events or an entry is NULL.
 */
#define STA_BWD_TIMED_EVENTS 5
sta_status sta_backward_timed(const sta_dims* dims, const void* q, const void* k,
                              const void* v, const void* out, const float* lse,
                              const void* dout, const int32_t* window_sizes,
                              int32_t text_length, int32_t has_text, void* dq, void* dk,
                              void* dv, void* workspace, size_t workspace_bytes,
                              void* stream, void* const* events);

#ifdef __cplusplus
}
#endif

#endif /* STA_H */
