/*
 * dp.h -- C ABI of libdp, the gfx950 (MI355X) library for one rank's share of
 * a displaced-patch (DistriFusion-style) diffusion step.
 *
 * The method (DistriFusion project summary, "How It Works"): the image is
 * split across devices; after a synchronous first step every device computes
 * its own rows fresh and takes the rest of the image from activations the
 * other devices produced one denoising step earlier.  Each device's rows are a
 * contiguous band of latent rows ("Benchmarking DistVAE", "Glossary":
 * patchify).  The three displaced layer kinds are self-attention, the 3x3
 * convolution and GroupNorm ("OTIL for SDXL on 4x L40S", "What is implemented
 * where"); their stale state is the attention K/V buffers, the conv halo rows
 * (same page, "Read this before interpreting the numbers", item 3) and two
 * scalars per GroupNorm group ("What is implemented where").
 *
 * Conventions for every call:
 *  - Activations are token-major, channels last: [B, T, C] with token
 *    t = row * W + col, so a rank's row band is one contiguous token range.
 *  - All tensor pointers are device memory owned by the caller; the library
 *    never allocates, frees or retains them.  Tensors are dense and
 *    contiguous in the stated layout.  Inputs and outputs must not overlap,
 *    except that dp_kv_buffer_splice updates its buffers in place.
 *  - Activations, weights and outputs of the bf16 GEMM/conv, bf16 attention
 *    and GroupNorm calls are moved in 16-byte pieces: their base pointers
 *    must be 16-byte aligned (torch allocations are; a slice that starts at a
 *    row boundary keeps it when a row is a multiple of 16 bytes), else
 *    DP_ERR_INVALID_ARG.  Statistics, gamma/beta and biases need only their
 *    element alignment.
 *  - `dt` is the storage type of every activation/weight tensor of a call.
 *    Statistics, GroupNorm gamma/beta and biases are always float32.
 *  - Calls are asynchronous: arguments are validated on the host first (a
 *    non-OK return has enqueued nothing and written nothing), then work is
 *    enqueued on `stream` and the call returns.  Faults during execution
 *    surface at the caller's next synchronisation of that stream.
 *  - State kept between calls, none of it caller data: the calling thread's
 *    last-error string; per device, a zero-filled 4 KiB device page the conv
 *    reads in place of absent halo rows and columns outside the image; per
 *    thread, the current device's CU count (asked again when the thread
 *    switches devices) and each device's resident attention blocks per CU
 *    (asked once); per device, the 4 MiB scratch
 *    of dp_groupnorm_stale_stats_noalloc and its address.  The environment
 *    variable DP_ATTN_SCHEDULE is read at every attention call and query.
 *    Calls on one stream are ordered; concurrent calls on different streams
 *    must not share output buffers or workspaces.
 */
#ifndef DP_H_
#define DP_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DP_OK = 0,
  DP_ERR_INVALID_ARG = 1, /* NULL required pointer, non-positive size, inconsistent shapes */
  DP_ERR_UNSUPPORTED = 2, /* valid arguments with no kernel for that shape/dtype */
  DP_ERR_HIP = 3          /* the HIP runtime reported an error at launch */
} dp_status;

/* DP_F16 (the latent's storage type on the pages) is accepted by the OTIL calls
 * only; every other call rejects it with DP_ERR_INVALID_ARG. */
typedef enum { DP_F32 = 0, DP_BF16 = 1, DP_F16 = 2 } dp_dtype;

/* Static description of a status code (never NULL). */
const char* dp_status_string(dp_status s);
/* Detail of the last non-OK return on the calling thread ("" if none). */
const char* dp_last_error(void);

/*
 * K/V buffer splice.  Stale state of a displaced self-attention layer is a
 * full-image K/V buffer per layer ("Tensor Parallelism with Stale
 * Activations ...", xDiT issue thread, maintainer's first reply: full spatial
 * shape K/V for every layer).  Each step the rank's own rows are replaced by
 * fresh values while every other row keeps its stale content; a position is
 * either fresh or stale, never a blend ("OTIL ...", "Self-tests").
 *
 * k_buf, v_buf     [B, T_kv, C], updated in place.
 * k_fresh, v_fresh [B, T_loc, C].
 * Tokens [t0, t0 + T_loc) of each batch item are overwritten bit for bit;
 * every other token is left untouched.  The copy is byte-exact for both dtypes.
 * Errors: INVALID_ARG for a NULL pointer, B/T_kv/C/T_loc <= 0, t0 < 0 or
 * t0 + T_loc > T_kv, or fresh rows overlapping the buffers.
 */
dp_status dp_kv_buffer_splice(void* k_buf, void* v_buf, const void* k_fresh, const void* v_fresh,
                              int64_t B, int64_t T_kv, int64_t C, int64_t t0, int64_t T_loc,
                              dp_dtype dt, hipStream_t stream);

/*
 * Attention of the rank's query rows over the whole spliced K/V buffer
 * ("OTIL ...", "What is implemented where": the displaced self-attention
 * layer; xDiT issue thread: fresh local and stale remote values mixed).
 * For each batch b, head h, query i:
 *   o = sum_j softmax_j(scale * <q_i, k_j>) v_j   over all T_kv keys, no mask.
 * Head h occupies channels [h*d, (h+1)*d) of the C = H*d channels.
 *
 * q     [B, Tq, H*d];  k_buf, v_buf [B, T_kv, H*d];  out [B, Tq, H*d].
 * scale <= 0 selects 1/sqrt(d).  Softmax and accumulation run in float32;
 * in bf16 the probabilities are rounded to bf16 before the P*V product.
 * q, k_buf and v_buf must hold finite values: the bf16 kernel fixes each
 * row's softmax reference from its first key block and moves it only when a
 * later block's row sum overflows, so a NaN or infinite input gives an
 * undefined output rather than a propagated NaN.
 * Supported: bf16 with d = 64; f32 with d in {32, 64}.
 * ws/ws_bytes: caller-owned device scratch of at least
 * dp_attn_stale_kv_workspace(...) bytes (NULL allowed when that is 0).  The
 * library picks one of two work schedules per shape (and per the device's CU
 * count); DP_ATTN_SCHEDULE=split or =balanced in the environment, read at
 * every call, forces one (tests and tuning).  The queried size covers both
 * schedules, so the setting never makes a queried workspace too small.
 * Errors: INVALID_ARG for NULL pointers, sizes <= 0 or a workspace that is too
 * small; UNSUPPORTED for other d or dtype combinations.
 */
size_t dp_attn_stale_kv_workspace(int64_t B, int64_t H, int64_t Tq, int64_t T_kv, int64_t d,
                                  dp_dtype dt);
dp_status dp_attn_stale_kv(const void* q, const void* k_buf, const void* v_buf, void* out,
                           int64_t B, int64_t H, int64_t Tq, int64_t T_kv, int64_t d, float scale,
                           dp_dtype dt, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * 3x3 convolution of the rank's rows whose missing neighbour rows come from
 * the stale halo buffers ("OTIL ...", "What is implemented where": the
 * displaced conv; "Benchmarking DistVAE", "Glossary": a halo is the
 * neighbouring rows a sharded convolution needs).  Stride 1, cross-correlation:
 *   y[b,i,x,o] = bias[o] + sum_{dy,dx in -1..1} sum_c w[o,dy+1,dx+1,c] * src(b,i+dy,x+dx,c)
 * where src row -1 is halo_top, row h is halo_bot, and columns outside
 * [0, W) are zero.
 *
 * x [B, h, W, Cin]; halo_top, halo_bot [B, W, Cin] or NULL (an image edge:
 * zeros); w [Cout, 3, 3, Cin]; bias [Cout] float32 or NULL; y [B, h, W, Cout].
 * Supported: bf16 with Cin % 32 == 0, Cin <= 2048 and Cout % 32 == 0 (MFMA path);
 * f32 any size.
 * Errors: INVALID_ARG for NULL x/w/y or sizes <= 0; UNSUPPORTED otherwise.
 */
dp_status dp_conv3x3_stale_halo(const void* x, const void* halo_top, const void* halo_bot,
                                const void* w, const float* bias, void* y,
                                int64_t B, int64_t h, int64_t W, int64_t Cin, int64_t Cout,
                                dp_dtype dt, hipStream_t stream);

/*
 * The displaced 3x3 convolution of dp_conv3x3_stale_halo, which also returns
 * the GroupNorm sums of its output, so the GroupNorm that follows needs no
 * read pass of its own to form them (the conv output feeds the displaced
 * GroupNorm, "OTIL ...", "What is implemented where").
 * y is exactly what dp_conv3x3_stale_halo writes.  gn_sums[b, g, :] =
 * (sum y, sum y^2) of the stored (bf16) outputs of batch item b over the h*W
 * tokens and the Cout/G channels of group g, float32, accumulated per output
 * tile in the conv epilogue and folded in a fixed order by a second launch
 * (deterministic; equal to dp_groupnorm_sums of y up to float32 rounding
 * order).
 * gn_sums [B, G, 2] float32; ws/ws_bytes: caller-owned device scratch of at
 * least dp_conv3x3_gn_sums_workspace(B, h, W, Cout) bytes for the tile
 * partials; its contents on entry do not matter, and calls that share it
 * must not overlap in time; other arguments as dp_conv3x3_stale_halo.
 * Supported: bf16 with Cin % 32 == 0, Cin <= 2048, Cout % 32 == 0,
 * Cout <= 2048 and h*W >= 160.  Errors: INVALID_ARG for NULL x/w/y/gn_sums, sizes <= 0,
 * Cout % G != 0, a short workspace or overlapping buffers; UNSUPPORTED
 * otherwise (f32 included: use dp_conv3x3_stale_halo then dp_groupnorm_sums).
 */
size_t dp_conv3x3_gn_sums_workspace(int64_t B, int64_t h, int64_t W, int64_t Cout);
dp_status dp_conv3x3_stale_halo_gn_sums(const void* x, const void* halo_top, const void* halo_bot,
                                        const void* w, const float* bias, void* y, float* gn_sums,
                                        int64_t G, void* ws, size_t ws_bytes, int64_t B, int64_t h,
                                        int64_t W, int64_t Cin, int64_t Cout, dp_dtype dt,
                                        hipStream_t stream);

/*
 * GroupNorm of the rank's tokens with statistics of the whole image: fresh
 * sums over the local tokens plus the stale sums the other patches produced
 * one step earlier ("OTIL ...", "What is implemented where": two scalars per
 * group decide slice brightness and contrast; "Manual runs": per-slice
 * statistics show as a contrast step at the seam; xDiT issue thread: partial
 * stale values).  For batch b and group g (channels [g*C/G, (g+1)*C/G)):
 *   S = (sum x, sum x^2 over local tokens) + sum_{p != rank} stale_sums[p,b,g,:]
 *   n = T_total * C/G;  mean = S0/n;  var = max(S1/n - mean^2, 0)
 *   y = (x - mean) / sqrt(var + eps) * gamma[c] + beta[c]   (then y*sigmoid(y) if fuse_silu)
 *
 * x [B, T_loc, C]; stale_sums [n_patches, B, G, 2] float32, entry [rank] is
 * never read; gamma, beta [C] float32 or NULL (1 and 0); y [B, T_loc, C];
 * fresh_sums_out [B, G, 2] float32 receives the local sums, or NULL.
 * ws/ws_bytes: at least dp_groupnorm_stale_stats_workspace(...) bytes,
 * zero-filled by the caller before its first use (its first 32 KiB hold
 * ticket counters that every call leaves at zero again, so one zero fill
 * serves any later calls and shapes, on one stream at a time).
 * Supported: C % G == 0, C % 8 == 0 (bf16) or C % 4 == 0 (f32), C <= 2048.
 * Errors: INVALID_ARG for NULL x/y/stale_sums (stale_sums may be NULL only
 * when n_patches == 1), sizes <= 0, rank outside [0, n_patches), T_total < T_loc,
 * eps < 0, C % G != 0, or a workspace that is too small.
 */
size_t dp_groupnorm_stale_stats_workspace(int64_t B, int64_t T_loc, int64_t C, int64_t G);
dp_status dp_groupnorm_stale_stats(const void* x, const float* stale_sums, int64_t n_patches,
                                   int64_t rank, int64_t T_total, const float* gamma,
                                   const float* beta, float eps, int fuse_silu, void* y,
                                   float* fresh_sums_out, int64_t B, int64_t T_loc, int64_t C,
                                   int64_t G, dp_dtype dt, void* ws, size_t ws_bytes,
                                   hipStream_t stream);

/*
 * dp_groupnorm_stale_stats without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, serving loops
 * that allocate nothing per call, harnesses that forbid hipMalloc).  Same
 * arguments (minus ws/ws_bytes), results and errors; the call allocates
 * nothing.  Its workspace is a static 4 MiB device array, one per device,
 * held until the process ends: shapes whose
 * dp_groupnorm_stale_stats_workspace(...) exceeds 4 MiB are rejected with
 * DP_ERR_UNSUPPORTED.  Every call on a device shares that device's array:
 * calls that overlap on one device (different streams, not ordered by the
 * caller) race and give wrong results.  The first call on a device also
 * looks up the array's address and enqueues a small fill kernel on `stream`
 * that zeroes its counters; a caller that captures the call in a HIP graph
 * makes one call before capturing, so that this set-up stays outside the
 * graph.
 */
dp_status dp_groupnorm_stale_stats_noalloc(const void* x, const float* stale_sums, int64_t n_patches,
                                           int64_t rank, int64_t T_total, const float* gamma,
                                           const float* beta, float eps, int fuse_silu, void* y,
                                           float* fresh_sums_out, int64_t B, int64_t T_loc, int64_t C,
                                           int64_t G, dp_dtype dt, hipStream_t stream);

/*
 * Local GroupNorm sums only: the first half of a GroupNorm whose statistics
 * are combined across row bands before normalising (DistVAE row mode,
 * "Benchmarking DistVAE", "Default suite", item 2: adapted layers work on
 * rank-local row bands; "OTIL ...", "What is implemented where": the two
 * scalars per group are what ranks exchange).  The sums are bit-identical to
 * the fresh_sums_out dp_groupnorm_stale_stats writes for the same x.
 *   sums_out[b, g, :] = (sum x, sum x^2) over the T_loc tokens and the C/G
 *   channels of group g, float32.
 * x [B, T_loc, C] of dt; sums_out [B, G, 2] float32; ws/ws_bytes as for
 * dp_groupnorm_stale_stats (dp_groupnorm_stale_stats_workspace).
 * Supported and errors: as dp_groupnorm_stale_stats (C % G == 0, C % 8 == 0 for
 * bf16 or C % 4 == 0 for f32, C <= 2048); INVALID_ARG also when sums_out
 * overlaps x or the workspace.
 */
dp_status dp_groupnorm_sums(const void* x, float* sums_out, int64_t B, int64_t T_loc, int64_t C,
                            int64_t G, dp_dtype dt, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * The normalising half of dp_groupnorm_stale_stats, with the rank's local sums
 * supplied by the caller (from dp_conv3x3_stale_halo_gn_sums or
 * dp_groupnorm_sums): one pass over x, no workspace.  Statistics, output and
 * SiLU as dp_groupnorm_stale_stats with S = local_sums + sum_{p != rank}
 * stale_sums[p]; given the sums dp_groupnorm_sums returns for x, y equals
 * dp_groupnorm_stale_stats's bit for bit.
 * local_sums [B, G, 2] float32; other arguments as dp_groupnorm_stale_stats.
 * Errors: as dp_groupnorm_stale_stats, plus INVALID_ARG for NULL local_sums.
 */
dp_status dp_groupnorm_apply(const void* x, const float* local_sums, const float* stale_sums,
                             int64_t n_patches, int64_t rank, int64_t T_total, const float* gamma,
                             const float* beta, float eps, int fuse_silu, void* y, int64_t B,
                             int64_t T_loc, int64_t C, int64_t G, dp_dtype dt, hipStream_t stream);

/*
 * Dense projection of the rank's own rows (the Q/K/V and output projections
 * inside the displaced self-attention layer; only local rows are projected,
 * stale rows are never recomputed):
 *   y[m, o] = sum_c x[m, c] * w[o, c] (+ bias[o])
 * x [M, Cin]; w [Cout, Cin]; bias [Cout] float32 or NULL; y [M, Cout].
 * Supported: bf16 with Cin % 32 == 0 and Cout % 32 == 0; f32 any size.
 * Errors: INVALID_ARG for NULL x/w/y or sizes <= 0; UNSUPPORTED otherwise.
 */
dp_status dp_linear(const void* x, const void* w, const float* bias, void* y, int64_t M,
                    int64_t Cin, int64_t Cout, dp_dtype dt, hipStream_t stream);

/*
 * Fused Q/K/V projection of the rank's rows, with K and V written straight
 * into the full-image buffers: the projections and the K/V splice in one
 * launch (the displaced attention's buffers hold the rank's fresh rows and
 * everyone else's stale rows: "OTIL ...", "What is implemented where"; xDiT
 * issue thread, maintainer's first reply).  For b in [0, B), i in [0, T_loc):
 *   q[b, i, :]          = x[b, i, :] . Wq^T
 *   k_buf[b, t0 + i, :] = x[b, i, :] . Wk^T
 *   v_buf[b, t0 + i, :] = x[b, i, :] . Wv^T
 * Every other row of k_buf and v_buf is left untouched.  Each value is the
 * one dp_linear computes (same reduction order), so the call equals three
 * dp_linear calls followed by dp_kv_buffer_splice, bit for bit.
 * x, q [B, T_loc, C]; wq, wk, wv [C, C]; k_buf, v_buf [B, T_kv, C]; no bias.
 * Supported: bf16 with C % 32 == 0; f32 any C.
 * Errors: INVALID_ARG for NULL pointers, sizes <= 0, t0 < 0 or
 * t0 + T_loc > T_kv, or outputs overlapping inputs or each other;
 * UNSUPPORTED for other shapes.
 */
dp_status dp_qkv_projection_into_buffers(const void* x, const void* wq, const void* wk,
                                         const void* wv, void* q, void* k_buf, void* v_buf,
                                         int64_t B, int64_t T_loc, int64_t T_kv, int64_t t0,
                                         int64_t C, dp_dtype dt, hipStream_t stream);

/*
 * OTIL selective block transmit, sender side: score, select and pack the
 * blocks of the rank's latent band that its peers receive this step ("OTIL for
 * SDXL on 4x L40S", "What is implemented where": one topk over the cosine
 * dissimilarity plus ten times an unvisited flag, packing by index select, no
 * host synchronisation; "Self-tests": exactly k blocks per peer).
 * Block j is the bh x bw spatial block (row-major over the (h/bh) x (W/bw)
 * block grid) of every batch item and channel.  Three kernels on `stream`:
 *   scores[j] = 1 - cos(x_j, last_sent_j) + (visited[j] ? 0 : bonus),
 *               cos = <a,b> / max(|a||b|, 1e-8), float32 accumulation;
 *   idx[0..k) = the k blocks of highest score, highest first, equal scores in
 *               block-id order (a NaN score ranks last);
 *   packed[p] = block idx[p] of x; last_sent's block idx[p] = that block of x;
 *               visited[idx[p]] = 1.
 * x, last_sent [B, h, W, C] of dt (F32, BF16 or F16); visited [K] uint8
 * (0/1, caller-owned state: clear it to start a new polling round); scores [K]
 * float32 out; idx [k] int32 out; packed [k, B, bh, bw, C] of dt out;
 * K = (h/bh)*(W/bw).  Pass bonus = 10 for the pages' rule (any value > 2 puts
 * unvisited blocks first).
 * Errors: INVALID_ARG for NULL pointers, sizes <= 0, h % bh or W % bw != 0,
 * k > K, a non-finite bonus, overlapping buffers or pointers not aligned to
 * their element size; UNSUPPORTED for K > 16384 or a band over 2 GiB.
 */
dp_status dp_otil_select_pack(const void* x, void* last_sent, uint8_t* visited, float* scores,
                              int32_t* idx, void* packed, int64_t B, int64_t h, int64_t W,
                              int64_t C, int64_t bh, int64_t bw, int64_t k, float bonus,
                              dp_dtype dt, hipStream_t stream);

/*
 * OTIL receiver side: copies each received block into the receiver's copy of
 * the sending peer's band, whole blocks only, so every position of that band
 * is either a received block or the previous (stale) content, never a blend
 * ("OTIL ...", "What is implemented where": one index copy per remote device;
 * "Self-tests").
 * dst [B, H, W, C] of dt, the receiver's copy of the whole latent, updated in
 * place; the peer's band is rows [r0, r0 + h).  packed [k, B, bh, bw, C] and
 * idx [k] int32 as produced by the peer's dp_otil_select_pack; ids outside
 * [0, K) are skipped.
 * Errors: INVALID_ARG for NULL pointers, sizes <= 0, r0 < 0 or r0 + h > H,
 * h % bh or W % bw != 0, k > K, dst overlapping packed or idx, or misaligned
 * pointers; UNSUPPORTED for a latent over 2 GiB.
 */
dp_status dp_otil_unpack(void* dst, const void* packed, const int32_t* idx, int64_t B, int64_t H,
                         int64_t W, int64_t C, int64_t r0, int64_t h, int64_t bh, int64_t bw,
                         int64_t k, dp_dtype dt, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* DP_H_ */
