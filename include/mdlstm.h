/*
 * mdlstm.h — C ABI of libmdlstm: example-packed 4-direction 2D MDLSTM on MI355X (gfx950).
 *
 * The method is that of "No Padding Please: Efficient Neural Handwriting
 * Recognition": variable-size images are tiled onto one 2D canvas with
 * separator pixels and a mask instead of being padded and stacked (§V), and a
 * 4-directional 2D MDLSTM layer (§III) runs over that canvas; the block-strided
 * convolution between MDLSTM levels works on chunked example lists (§V-B).
 *
 * Conventions for every entry point below
 *  - Plain C types only. Device pointers are HIP device memory owned by the
 *    caller; the library never allocates or frees device memory. Host pointers
 *    are marked "host".
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Device
 *    work is enqueued asynchronously on it; nothing synchronizes unless stated.
 *  - Return value: MDL_OK or a negative MDL_E* code; on failure nothing has been
 *    launched or written and mdl_last_error() holds a message (thread-local,
 *    valid until the next call on that thread). The library never prints and
 *    never aborts. A device fault inside a kernel surfaces at the caller's next
 *    synchronization, as for any HIP work.
 *  - Outputs are overwritten, never accumulated into.
 *  - Results are deterministic: the same inputs on the same stream give
 *    bit-identical outputs (fixed reduction orders, no floating-point atomics).
 *
 * Canvas conventions
 *  - The canvas is Hc x Wc pixels, row-major. Channel-last tensors on it are
 *    [Hc][Wc][K]; per-direction tensors are [4][Hc][Wc][H] (direction-major).
 *  - Directions: 0 scans from the top-left, 1 from the top-right, 2 from the
 *    bottom-left, 3 from the bottom-right. For direction (sy, sx) in
 *    {(+1,+1), (+1,-1), (-1,+1), (-1,-1)} the predecessors of (y, x) are
 *    "left" (y, x - sx) and "up" (y - sy, x) ("as defined by the scanning
 *    direction", §IV-A).
 *  - Per-example ("flat") tensors are the examples' [h][w][K] blocks
 *    concatenated in input order.
 *  - Gate axis of width 5H, in blocks of H: (i, f_left, f_up, o, g).
 *    Wx[4][C][5H], Ul[4][H][5H], Uu[4][H][5H], b[4][5H], all float32.
 */
#ifndef MDLSTM_H
#define MDLSTM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define MDL_OK            0
#define MDL_EINVAL       (-1) /* bad argument (null pointer, non-positive size, bad enum) */
#define MDL_ENOMEM       (-2) /* host allocation failed */
#define MDL_EOVERFLOW    (-3) /* canvas or buffer size exceeds the 32-bit index range */
#define MDL_ESIZE        (-4) /* caller buffer (workspace, descriptor) too small */
#define MDL_EHIP         (-5) /* HIP runtime or launch error */
#define MDL_EUNSUPPORTED (-6) /* size combination this build does not handle (e.g. LDS limit) */

/* packing modes */
#define MDL_PACK_ALG1   0 /* shelf packing, §IX-B (packing algorithm details, Algorithm 1) */
#define MDL_PACK_PADDED 1 /* minimal per-batch padding ("batch-padding", §VII-C) */
#define MDL_PACK_EXACT  2 /* shelf packing with exact-height rows (§V, §V-A prose) */

/* element types of pixel tensors */
#define MDL_F32  0
#define MDL_BF16 1

/* cells ("No Padding Please" §III) */
#define MDL_CELL_MDLSTM   0 /* the 2D MDLSTM cell: input gate, two forget gates, output gate */
#define MDL_CELL_LEAKY_LP 1 /* the stable Leaky LP cell: lambda gate, leaky update, two output gates */

/* indices into the int64 array filled by mdl_layout_info */
#define MDL_INFO_N              0 /* examples */
#define MDL_INFO_CANVAS_H       1
#define MDL_INFO_CANVAS_W       2
#define MDL_INFO_ROWS           3 /* packed rows (padded mode: n) */
#define MDL_INFO_REAL_PIXELS    4 /* sum of h*w */
#define MDL_INFO_COMPUTED_CELLS 5 /* cells the MDLSTM computes per direction (padded mode: n*Hmax*Wmax) */
#define MDL_INFO_MAX_DEPTH      6 /* max over examples of h+w-1: dependent steps per pass */
#define MDL_INFO_MAX_DIAG       7 /* max over examples of min(h,w): widest anti-diagonal */
#define MDL_INFO_MODE           8
#define MDL_INFO_WG_GROUPS      9 /* groups of the weight-gradient split (one task per group and direction) */
#define MDL_INFO_COUNT         10

typedef struct mdl_layout mdl_layout; /* host object, immutable once built */

/*
 * mdl_pack — place n examples of sizes heights[e] x widths[e] (host arrays) on a
 * canvas. Host-only, integer, allocates only the returned layout.
 *
 * MDL_PACK_ALG1 (§V, §V-A, §IX-B (packing algorithm details, Algorithm 1)): canvas width
 * Wc = max(canvas_w_min, max width); examples are bucketed by height and the
 * buckets visited tallest first; rows are filled with the widest example of the
 * current bucket that still fits (ties: lowest index), `sep` separator pixels
 * between neighbours; a row is closed only when nothing of the current bucket
 * fits, so it may continue into the next, shorter bucket; rows are stacked
 * with `sep` separator rows between them, examples top-aligned. The skew of
 * Algorithm 1's last step is not applied (it changes no cell's value).
 * MDL_PACK_PADDED (§VII-C, batch padding): slot e at (e*Hmax, 0) of size
 * Hmax x Wmax, the real pixels top-left; every slot cell is computed.
 * MDL_PACK_EXACT (§V: the examples of one packed row share one height, as the
 * input-skewing trick of §IV-A requires; §V-A step 2 fills rows inside each
 * height bucket): as MDL_PACK_ALG1, but a row is also closed when its bucket
 * is used up, so no row mixes heights. The kernels compute the same cells
 * (the real pixels) in every packed mode; only the canvas differs.
 *
 * Errors: MDL_EINVAL for n < 1, null pointers, a size < 1, sep < 0,
 * canvas_w_min < 1 or an unknown mode; MDL_EOVERFLOW if Hc*Wc >= 2^31;
 * MDL_ENOMEM. On success *out owns the layout (free with mdl_layout_free).
 */
int mdl_pack(const int32_t* heights, const int32_t* widths, int32_t n, int32_t canvas_w_min,
             int32_t sep, int32_t mode, mdl_layout** out);

/*
 * mdl_pack_level — the layout of the next MDLSTM level of a stack ("No Padding
 * Please" §V-B: a block-strided convolution of kh x kw blocks between two
 * MDLSTM levels lowers each example's resolution, and the examples are packed
 * again just before the next MDLSTM layer). Example e of the new layout has
 * ceil(h_e / kh) x ceil(w_e / kw) cells, (h_e, w_e) its size in `lk` (the last
 * row and column of blocks are zero-padded), examples in the same order; the
 * sizes are then packed as by mdl_pack(..., canvas_w_min, sep, mode, out).
 * Host-only; `lk` is only read. Errors: those of mdl_pack, and MDL_EINVAL for
 * a null `lk` or `out` or kh, kw < 1.
 */
int mdl_pack_level(const mdl_layout* lk, int32_t kh, int32_t kw, int32_t canvas_w_min, int32_t sep,
                   int32_t mode, mdl_layout** out);

/* Frees a layout from mdl_pack or mdl_pack_level (NULL is ignored). */
void mdl_layout_free(mdl_layout* layout);

/* Fills info[MDL_INFO_COUNT] (host) with the layout's sizes. */
int mdl_layout_info(const mdl_layout* layout, int64_t* info);

/*
 * Host copies of the rectangles, input order, as [n][4] = (y0, x0, h, w):
 * `rects` the computed region of each example, `real` its real pixels (equal
 * in the two shelf modes). Either pointer may be NULL.
 */
int mdl_layout_rects(const mdl_layout* layout, int32_t* rects, int32_t* real);

/*
 * The unit schedule: the wavefront kernels run one workgroup per (example,
 * direction) unit, u = 4*e + d, and workgroup i takes units[i] (host array of
 * 4n entries; the units with the most cells first, so the longest chains start
 * first). *desc_offset receives the byte offset of this int32 array in the
 * device descriptor that mdl_layout_upload writes. Results do not depend on
 * the order (each unit's arithmetic is fixed and every reduction runs in a
 * fixed order); a caller may permute the array in an uploaded descriptor, which
 * only changes the dispatch order. Errors: MDL_EINVAL for a null argument.
 */
int mdl_layout_units(const mdl_layout* layout, int32_t* units, size_t* desc_offset);

/*
 * Original example indices per packed row (Algorithm 1's result): row r holds
 * row_examples[row_start[r] .. row_start[r+1]-1], left to right.
 * row_start has info[MDL_INFO_ROWS]+1 entries, row_examples n.
 */
int mdl_layout_rows(const mdl_layout* layout, int32_t* row_start, int32_t* row_examples);

/*
 * Host per-pixel maps (§V: the binary mask, here with the example id): eid[Hc*Wc]
 * = example covering the pixel's computed region or -1; border[Hc*Wc] bit 0/1/2/3
 * set when the neighbour (y,x-1)/(y,x+1)/(y-1,x)/(y+1,x) belongs to the same
 * example. A predecessor whose bit is clear reads as zero hidden and memory state.
 */
int mdl_layout_maps(const mdl_layout* layout, int32_t* eid, uint8_t* border);

/*
 * Size of the device descriptor of a layout (rects, offsets, unit schedule and
 * the device eid/border maps), and the byte offsets of the eid (int32) and
 * border (uint8) maps inside it.
 */
int mdl_layout_device_size(const mdl_layout* layout, size_t* bytes, size_t* eid_offset,
                           size_t* border_offset);

/*
 * Copies the layout's descriptor into d_desc (device, >= the size above) and
 * builds the eid/border maps there with a kernel. Synchronizes `stream` before
 * returning, so the layout may be freed afterwards. MDL_ESIZE if bytes is too small.
 */
int mdl_layout_upload(const mdl_layout* layout, void* d_desc, size_t bytes, void* stream);

/*
 * Workspace bytes mdl_forward/mdl_backward need for a layer with C input channels
 * and H hidden units per direction on this layout: the forward stash (gates and
 * memory state of every computed cell), the projection / gate-gradient buffer
 * and the weight-gradient partial sums. The same workspace must be passed,
 * unmodified, from mdl_forward to the mdl_backward that follows it.
 */
int mdl_workspace_size(const mdl_layout* layout, int32_t C, int32_t H, size_t* bytes);

/*
 * Scatter ("No Padding Please" §V-A, step 3: the examples are tiled onto the
 * packed canvas at the positions the packer chose, separator and unused pixels
 * zero): x_flat (device, flat [h][w][C] per example, input order, dtype MDL_F32
 * or MDL_BF16) -> x_canvas (device, [Hc][Wc][C], same dtype), zero outside the
 * real pixels (separators, unused canvas, padding). Bit-exact copy.
 * Errors: MDL_EINVAL for null pointers, C < 1 or an unknown dtype; MDL_EHIP
 * for a launch failure. Asynchronous on `stream`.
 */
int mdl_scatter(const mdl_layout* layout, const void* d_desc, const void* x_flat, int32_t C,
                int32_t dtype, void* x_canvas, void* stream);

/*
 * Forward of one 4-direction MDLSTM layer over the canvas.
 * Input projection x.Wx + b of every computed cell and direction (§IV-B: the
 * five input matrices computed together; RETURNN §4.2: the non-recurrent part
 * as one matrix product), formed on the matrix cores inside the wavefront step
 * for the hidden sizes and channel counts the library instantiates and as one
 * GEMM before it otherwise, and the recurrence as an anti-diagonal wavefront
 * (§I; RETURNN §4.2: all positions of a diagonal at once, four directions at
 * once), each example on its own local diagonals. `cell`:
 *   MDL_CELL_MDLSTM (§III, Figure 4(a)): Vl and Vu must be NULL;
 *     a = x.Wx[d] + b[d] + h_left.Ul[d] + h_up.Uu[d]      (gates i, f_l, f_u, o, g)
 *     i, f_l, f_u, o = sigmoid(.), g = tanh(.)
 *     c = f_l*c_left + f_u*c_up + i*g,  h = o*tanh(c)
 *   MDL_CELL_LEAKY_LP (§III, Figure 4(b), §IX-A): Vl, Vu [4][H][3H] project the
 *   predecessors' memory states onto the gates lam, o1, o2;
 *     a = x.Wx[d] + b[d] + h_left.Ul[d] + h_up.Uu[d]      (gates f, lam, o1, o2, g)
 *     a[lam, o1, o2] += s_left.Vl[d] + s_up.Vu[d]
 *     sbar = lam*s_left + (1-lam)*s_up,  s = f*sbar + (1-f)*g,  h = o1*tanh(s) + o2*s
 *   (supported for H in {4, 8, 16, 32}, C <= 16, and a widest diagonal of at
 *   most 64 cells, 32 at H = 32; MDL_EUNSUPPORTED otherwise).
 * Predecessors outside the example read as zero (§V mask).
 * x_canvas [Hc][Wc][C] (x_dtype), h_dirs out [4][Hc][Wc][H] float32 (zero
 * outside the computed region). ws: >= mdl_workspace_size bytes.
 * MDL_EINVAL for an unknown cell, or Vl/Vu given with the plain cell or missing
 * with the Leaky LP one. MDL_EUNSUPPORTED when H or the widest diagonal exceed
 * the kernel's LDS budget, or when one direction's h plane (Hc*Wc*H floats) or
 * the canvas input exceeds 1 GiB (buffer ranges are 32-bit).
 */
int mdl_forward(const mdl_layout* layout, const void* d_desc, const void* x_canvas, int32_t x_dtype,
                int32_t C, int32_t H, int32_t cell, const float* Wx, const float* Ul, const float* Uu,
                const float* b, const float* Vl, const float* Vu, float* h_dirs, void* ws,
                size_t ws_bytes, void* stream);

/*
 * mdl_forward followed by mdl_dirsum_unpack (the layer output: the four
 * directions' h added in direction order and un-packed to the flat per-example
 * layout, "No Padding Please" §III, §V-A), in one call. y_flat [sum h*w][H]
 * float32, flat per example in input order, must not be NULL. When the
 * wavefront's (example, direction) units leave at least half of the device's
 * compute units free (f16 wavefront, H a multiple of 4, 16-byte aligned h_dirs
 * and y_flat), the direction sum overlaps the wavefront: each unit flags itself
 * once its h plane is stored, workgroups on the library's own stream (as in
 * mdl_backward) sum the output in runs of at most 256 pixels of one example,
 * in the order the examples finish, once all four of an example's units are
 * done, and a launch on `stream` after the wavefront takes the runs they did
 * not get to. Every run is summed by the same code whichever launch takes it,
 * so y equals mdl_dirsum_unpack's bit for bit. Every wait is bounded, and
 * mdl_set_wgrad_overlap's mode applies to this overlap as well. Arguments and
 * errors otherwise as mdl_forward; ws: >= mdl_workspace_size bytes.
 */
int mdl_forward_dirsum(const mdl_layout* layout, const void* d_desc, const void* x_canvas, int32_t x_dtype,
                       int32_t C, int32_t H, int32_t cell, const float* Wx, const float* Ul, const float* Uu,
                       const float* b, const float* Vl, const float* Vu, float* h_dirs, float* y_flat,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * The pages' own schedule of the recurrence, for comparison with the local
 * diagonals of mdl_forward / mdl_backward ("No Padding Please" §IV-A, Figure 3:
 * the whole packed canvas skewed, row i shifted right by i, and computed one
 * skewed column after another; RETURNN §4.2: one kernel launch per diagonal).
 * A pass takes Hc + Wc - 1 dependent column steps, one launch each (all four
 * directions in it), and every cell of the skewed grid is computed, padding
 * and separators included, with only the example cells kept (§V mask). The
 * results are the same cells as mdl_forward / mdl_backward's with
 * MDL_CELL_MDLSTM (fp32 arithmetic, not the same rounding), in the same
 * layouts: h_dirs, and the workspace's stash and gate gradients, so the
 * weight gradients come from the same kernels. Arguments as mdl_forward /
 * mdl_backward with the plain cell; the workspace is at least
 * mdl_skewed_workspace_size bytes (mdl_workspace_size plus the dc f_l, dc f_u
 * products every cell sends to its predecessors, 8H bytes per cell and
 * direction), carried from mdl_forward_skewed to mdl_backward_skewed.
 * MDL_EUNSUPPORTED for H outside {4, 16}; other errors as mdl_forward /
 * mdl_backward.
 */
int mdl_skewed_workspace_size(const mdl_layout* layout, int32_t C, int32_t H, size_t* bytes);
int mdl_forward_skewed(const mdl_layout* layout, const void* d_desc, const void* x_canvas,
                       int32_t x_dtype, int32_t C, int32_t H, const float* Wx, const float* Ul,
                       const float* Uu, const float* b, float* h_dirs, void* ws, size_t ws_bytes,
                       void* stream);
int mdl_backward_skewed(const mdl_layout* layout, const void* d_desc, const void* x_canvas,
                        int32_t x_dtype, int32_t C, int32_t H, const float* Wx, const float* Ul,
                        const float* Uu, const float* h_dirs, const float* dy_flat,
                        const float* dh_dirs, float* dx_flat, float* dx_canvas, float* dWx,
                        float* dUl, float* dUu, float* db, void* ws, size_t ws_bytes, void* stream);

/*
 * Direction sum and un-packing (§III four directions combined; §V-A
 * un-packing by original index and size, separators dropped):
 * y_flat[e][r][c][k] = sum_{d=0..3} h_dirs[d][y0+r][x0+c][k] over each real pixel,
 * summed in the order d = 0,1,2,3.
 */
int mdl_dirsum_unpack(const mdl_layout* layout, const void* d_desc, const float* h_dirs,
                      int32_t H, float* y_flat, void* stream);

/*
 * 2D BPTT backward of the mdl_forward that filled `ws` (RETURNN §4.2: the
 * recurrent part back-propagated over the diagonals in reverse, then the
 * weight and input gradients as matrix products), for the same `cell`.
 * Upstream gradient: exactly one of
 *   dy_flat  (flat [h][w][H], gradient of the direction-summed output; every
 *            direction receives it), or
 *   dh_dirs  ([4][Hc][Wc][H], gradient of each direction's output).
 * Outputs (each may be NULL except the weight gradients):
 *   dx_flat [h][w][C] float32 per example, dx_canvas [Hc][Wc][C] float32 (zero
 *   outside the real pixels); dWx, dUl, dUu, db shaped like Wx, Ul, Uu, b; for
 *   MDL_CELL_LEAKY_LP also dVl, dVu shaped like Vl, Vu (NULL, with Vl and Vu,
 *   for the plain cell).
 * Weight gradients are fixed-order blocked sums over all computed cells.
 * When the reverse wavefront's (example, direction) units leave at least half
 * of the device's compute units free (and the f16 wavefront and the
 * weight-gradient kernel cover H, C and the input type), the weight gradient
 * overlaps the wavefront: every unit counts itself on its example when its
 * gate gradients are stored, and persistent workgroups on a stream of the
 * library's own (one per device, forked from and joined back into `stream`
 * with events) take weight-gradient blocks from a claim queue, in the order
 * their examples finish, once those examples are done; after the wavefront a
 * launch on `stream` takes the rest of the queue on every compute unit while
 * they finish theirs, and a block given up beside the wavefront (each wait is
 * bounded) is computed after both. Each block is computed by the same code
 * whichever launch takes it, so the results are the same bit for bit.
 * Overlapping calls on one device share that stream (and a workspace must not
 * be shared by calls that may overlap).
 * MDL_EUNSUPPORTED under the same size limits as mdl_forward and when one
 * direction's gate gradients (T*5H floats, T = computed cells) reach 2 GiB.
 */
int mdl_backward(const mdl_layout* layout, const void* d_desc, const void* x_canvas, int32_t x_dtype,
                 int32_t C, int32_t H, int32_t cell, const float* Wx, const float* Ul, const float* Uu,
                 const float* Vl, const float* Vu, const float* h_dirs, const float* dy_flat,
                 const float* dh_dirs, float* dx_flat, float* dx_canvas, float* dWx, float* dUl,
                 float* dUu, float* db, float* dVl, float* dVu, void* ws, size_t ws_bytes, void* stream);

/*
 * Block-strided convolution between MDLSTM levels (§V-B), kernel kh x kw with
 * stride kh x kw, as one gather-GEMM over all blocks of all examples:
 *   x_k1[e][r][c][o] = bc[o] + sum_{d,k,i,j} Wc[o][d][k][i][j] * h_k[d][2r+i][4c+j][k]
 * (for kh=2, kw=4), where out-of-range input rows/cols read as zero. The
 * level-k layout `lk` gives where example e's level-k outputs are; the
 * level-(k+1) layout `lk1` must hold e with size ceil(h/kh) x ceil(w/kw) and
 * receives x_canvas_k1 [Hc'][Wc'][Cout] float32 (zero outside real pixels).
 * h_dirs_k [4][Hc][Wc][H]; Wc [Cout][4][H][kh][kw]; bc [Cout].
 * MDL_EUNSUPPORTED when Wc plus one tile of 16 blocks (floats: (Cout + 16) *
 * 4*H*kh*kw) exceeds a workgroup's LDS.
 */
int mdl_blockconv_forward(const mdl_layout* lk, const void* d_desc_k, const mdl_layout* lk1,
                          const void* d_desc_k1, const float* h_dirs_k, int32_t H, int32_t kh,
                          int32_t kw, const float* Wc, const float* bc, int32_t Cout,
                          float* x_canvas_k1, void* stream);

/* Workspace bytes for mdl_blockconv_backward (weight-gradient partial sums). */
int mdl_blockconv_workspace_size(const mdl_layout* lk1, int32_t H, int32_t kh, int32_t kw,
                                 int32_t Cout, size_t* bytes);

/*
 * Backward of mdl_blockconv_forward: dx_canvas_k1 [Hc'][Wc'][Cout] -> dh_dirs_k
 * [4][Hc][Wc][H] (zero outside the level-k real pixels), dWc, dbc (fixed-order
 * sums: partial sums over chunks of level-(k+1) canvas pixels, added in chunk
 * order). MDL_EUNSUPPORTED when Cout*(4*H*kh*kw+1) exceeds 8192, or when one
 * tile of 16 blocks and their output gradients, or Wc, exceeds a workgroup's LDS.
 */
int mdl_blockconv_backward(const mdl_layout* lk, const void* d_desc_k, const mdl_layout* lk1,
                           const void* d_desc_k1, const float* h_dirs_k, int32_t H, int32_t kh,
                           int32_t kw, const float* Wc, int32_t Cout, const float* dx_canvas_k1,
                           float* dh_dirs_k, float* dWc, float* dbc, void* ws, size_t ws_bytes,
                           void* stream);

/*
 * mdl_blockconv_backward without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops that forbid
 * allocation): the same computation and results as mdl_blockconv_backward,
 * with the weight-gradient partial sums in a fixed scratch array inside the
 * library, one per device, 16 MiB (the partials of any call that
 * mdl_blockconv_backward accepts: at most 512 chunks of Cout*(4*H*kh*kw+1) <=
 * 8192 floats). The array is held for the life of the process; its device
 * address is looked up on the first call on each device. Nothing is allocated
 * (no hipMalloc, no allocating library call). Every call on one device shares
 * that array: calls that overlap on one device (two streams, two threads)
 * race and must be serialized by the caller. Every partial is overwritten by
 * each call, so no clearing is needed between calls.
 * Errors: those of mdl_blockconv_backward; MDL_ESIZE if the partials would
 * exceed the scratch (no accepted call does); MDL_EHIP if the scratch's
 * address cannot be obtained.
 */
int mdl_blockconv_backward_noalloc(const mdl_layout* lk, const void* d_desc_k, const mdl_layout* lk1,
                                   const void* d_desc_k1, const float* h_dirs_k, int32_t H, int32_t kh,
                                   int32_t kw, const float* Wc, int32_t Cout, const float* dx_canvas_k1,
                                   float* dh_dirs_k, float* dWc, float* dbc, void* stream);

/*
 * Model head after the last MDLSTM level ("No Padding Please" §II / Figure 1:
 * one fully-connected layer shared across the four directions, trained with
 * CTC, the pages' reference [13]). For each example e of the layout, with
 * y_e = y_flat's [h][w][H] block (the direction sum, as mdl_dirsum_unpack
 * writes it):
 *   frames     Y[t][j] = sum over rows r of y_e[r][t][j], t < w (height collapse)
 *   logits     z[t][k] = sum_j Y[t][j] Wfc[j][k] + bfc[k], k < K, class 0 = blank
 *   loss[e]    = -ln p(l_e | z), the CTC probability of label l_e under the
 *                per-frame softmax of z (forward-backward recursion in log space)
 * and the gradients of sum_e loss[e]: dy_flat (every row of a frame receives
 * that frame's dz.Wfc^T), dWfc [H][K], dbfc [K].
 * Labels (device, int32): example e's label is labels[label_off[e] ..
 * label_off[e+1]-1], classes 1..K-1; label_off has n+1 entries; n_labels is
 * the length of `labels`; max_label bounds every label's length and sizes the
 * workspace. An example whose label cannot be aligned to its w frames gets
 * loss +inf and no gradient; one whose offsets leave [0, n_labels], decrease,
 * or whose label is longer than max_label or holds a class outside 1..K-1
 * gets loss NaN and no gradient (these are found on the device).
 * dy_flat may be NULL; dWfc and dbfc are both given or both NULL. dWfc / dbfc
 * are fixed-order sums (per-example partials added in example order).
 * ws: >= mdl_ctc_workspace_size bytes, device, contents not kept.
 * Errors: MDL_EINVAL for null tensors or H < 1, K < 2, max_label < 0;
 * MDL_EUNSUPPORTED for H > 1024, K > 4096 or max_label > 65535; MDL_EOVERFLOW
 * when the widest example's frames times max(H, K, 2 max_label + 1) reach 2^31;
 * MDL_ESIZE for a short workspace.
 */
int mdl_ctc_workspace_size(const mdl_layout* layout, int32_t H, int32_t K, int32_t max_label, size_t* bytes);
int mdl_ctc_head(const mdl_layout* layout, const void* d_desc, const float* y_flat, int32_t H,
                 const float* Wfc, const float* bfc, int32_t K, const int32_t* labels,
                 const int32_t* label_off, int64_t n_labels, int32_t max_label, float* loss,
                 float* dy_flat, float* dWfc, float* dbfc, void* ws, size_t ws_bytes, void* stream);

/*
 * Kernel timing (measurement support). mdl_timing(1) makes every later launch
 * of a kernel group (names: "build_maps", "scatter", "zero_fill", "projection",
 * "fwd_wavefront", "dirsum_overlap" (on the library's own stream, concurrent with
 * "fwd_wavefront"), "dirsum", "bwd_wavefront", "wgrad_overlap" (on the library's
 * own stream, concurrent with "bwd_wavefront"), "wgrad", "conv_fwd", "conv_bwd",
 * "ctc_head")
 * hand each of its dispatches a HIP event pair that the dispatch itself
 * records (hipExtLaunchKernel): the group's time runs from its first
 * dispatch's start to its last one's end, with no marker packets between
 * kernels. mdl_timing(0) stops recording. mdl_timing_only(name) limits the
 * recording to one group (NULL or "" restores all groups); every recorded
 * dispatch still costs the stream a few microseconds, so a throughput
 * measurement times only the group it needs. mdl_timing_report synchronizes
 * the recorded events and writes, for up to `max` kernel groups, the name
 * (NUL-terminated, 32 bytes per entry in `names`), the summed milliseconds and
 * the launch count; *count receives the number of groups; the records are then
 * cleared. Process-wide, not meant for concurrent use from several threads.
 * Errors: MDL_EINVAL for bad arguments or a name of 32 bytes or more.
 */
int mdl_timing(int32_t enable);
int mdl_timing_only(const char* group);

/* Sets the overlaps with the wavefronts, process-wide: the weight gradients beside the reverse wavefront
 * (mdl_backward) and the direction sum beside the forward one (mdl_forward_dirsum). 1 on (default), 0 off,
 * 2 on with no time allowed for any wait (every task or run claimed beside a wavefront is given up there and
 * computed after it: the path a wait that runs out of time takes, for tests). The results do not depend on
 * it. MDL_EINVAL for any other mode. */
int mdl_set_wgrad_overlap(int32_t mode);
int mdl_timing_report(int32_t max, char* names, double* total_ms, int64_t* launches, int32_t* count);

/* Message of the last failed call on this thread ("" if none). */
const char* mdl_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MDLSTM_H */
