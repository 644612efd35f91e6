/*
 * wq.h - C ABI of the MI355X (gfx950) group-wise low-bit weight-only GEMV library.
 *
 * Two weight formats, both grouped by 32 consecutive input channels (K):
 *
 *   W4: asymmetric uniform 4-bit grid, one FP16 scale s and one FP16 zero point
 *       z (an integer 0..15 stored as FP16) per (row, group).  Reconstruction
 *       w_hat = (q - z) * s.  Source: the SPECTRA page ("Compress Any LLM 3x in
 *       One Click, Near-Lossless in Under 50 MB RAM"), section 3.4
 *       "Microscaled Group-32 Quantization with Marlin-Interleaved Layout".
 *   W2: 2-bit codes into the FP16 Lloyd-Max codebook C = {-1.52, -0.45, +0.45,
 *       +1.52}, one FP16 scale S and zero Z per (row, group) fitted by ordinary
 *       least squares.  Reconstruction w_hat = S * C[q] + Z.  Source: the
 *       OTF-LLM v4.0 page (pypi otf-llm 4.0.0), sections 2, 3 and 5.
 *
 *   W4P: W4 with its zero points stored packed, two 4-bit zero points of
 *       adjacent groups per byte (SPECTRA section 3.4, "PackedZero"), 4.625
 *       instead of 5 bits per weight.  Same codes, scales and values as W4.
 *
 * In both formats a sorted set of n_out input channels (outlier columns) is kept
 * exactly in FP16 and added in the same kernel launch (SPECTRA section 4.1,
 * OTF-LLM "Architecture & Key Innovations": FP16 outliers plus quantized
 * background).  The quantized background skips those columns.
 *
 * Layouts (row-major, N output rows, K input channels, G = K / 32 groups):
 *   codes W4  uint8 [N][K/2]   byte 16g+k of row n = q[n][32g+k] | q[n][32g+16+k] << 4,
 *                              k = 0..15 (in-group nibble interleave, SPECTRA 3.4)
 *   codes W2  uint8 [N][K/4]   byte j of row n = q[4j] | q[4j+1]<<2 | q[4j+2]<<4 | q[4j+3]<<6
 *                              (OTF-LLM section 5)
 *   scales    uint16 (FP16 bits) [N][G]
 *   zeros     uint16 (FP16 bits) [N][G]   (W4, W2)
 *   zeros W4P uint8 [N][ceil(G/2)]   byte m of row n = z[n][2m] | z[n][2m+1] << 4
 *                              (the high nibble of the last byte is 0 when G is odd);
 *                              entry points that take `const uint16_t* zeros` read
 *                              these bytes through that pointer when fmt is WQ_FMT_W4P
 *   out_idx   int32  [n_out], strictly increasing, each in [0, K)
 *   out_w     uint16 (FP16 bits) [N][n_out]   out_w[n][j] = W[n][out_idx[j]]
 *   x / X     uint16 (FP16 bits) [M][K];  y / Y  uint16 (FP16 bits) [M][N]
 *
 * Conventions
 *   - Every function returns WQ_OK (0) or a negative WQ_ERR_* code; the message
 *     of the last error on the calling thread is wq_last_error().  Nothing
 *     aborts or throws across the ABI.
 *   - The caller allocates and frees every buffer.  The library allocates no
 *     device memory, keeps no workspace and no global state beyond its kernels.
 *   - Device entry points take device pointers and a HIP stream (hipStream_t
 *     passed as void*; NULL = the null stream).  They only enqueue work and never
 *     synchronize; a launch failure is reported as WQ_ERR_HIP.  Host entry points
 *     are synchronous and touch no GPU.
 *   - Supported shapes: N >= 1, 32 <= K <= 65536, K % 32 == 0, group == 32
 *     (any other group size is WQ_ERR_UNSUPPORTED), 0 <= n_out <= K.  Device
 *     pointers must be 16-byte aligned.  A pointer may be NULL only when the
 *     array it names is empty.
 *   - Device results are bit-reproducible from run to run (no atomics).
 */
#ifndef WQ_H
#define WQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WQ_OK 0
#define WQ_ERR_INVALID_ARG (-1)
#define WQ_ERR_UNSUPPORTED (-2)
#define WQ_ERR_HIP (-3)

#define WQ_FMT_W4 4
#define WQ_FMT_W2 2
#define WQ_FMT_W4P 5 /* W4 with packed 4-bit zero points */

/* flags of the product entry points */
#define WQ_FUSE_OUTLIERS 1u /* add the FP16 outlier columns inside the same launch */

#define WQ_GROUP 32
#define WQ_MAX_K 65536
#define WQ_GEMM_MAX_M 16

/* Text of a status code.  Never NULL. */
const char* wq_status_str(int status);
/* Message of the last failing call on this thread ("" if none).  Never NULL. */
const char* wq_last_error(void);
/* Library version string. */
const char* wq_version(void);

/* ------------------------------------------------------------------ host (CPU)
 * All host functions are synchronous, single-threaded, deterministic, and are
 * the reference encoders of the formats above.
 */

/* W4 quantize + pack (SPECTRA section 3.4, codes per Appendix A Proposition 2).
 * W: float32 [N][K] (typically the dense residual from wq_split_outliers).
 * Per (row, group), in float32 with round-half-to-even:
 *   s = max((wmax - wmin) / 15, 1e-8);  z = clamp(round(-wmin / s), 0, 15);
 *   q = clamp(round(w / s + z), 0, 15)   (codes use s before its FP16 rounding)
 * Outputs: codes [N][K/2] (layout above), scales = FP16(s), zeros = FP16(z).
 * Errors: WQ_ERR_INVALID_ARG for NULL pointers or bad N/K; WQ_ERR_UNSUPPORTED if
 * group != 32 or K % 32 != 0. */
int wq_quantize_w4(const float* W, int64_t N, int64_t K, int32_t group,
                   uint8_t* codes, uint16_t* scales, uint16_t* zeros);

/* W2 quantize + pack (OTF-LLM v4.0 sections 2, 3, 5), float64 per group of 32:
 * mean mu, population std sigma, u = (w - mu) / sigma (0 if sigma == 0), code
 * q = nearest FP16 centroid of u (ties to the lower code), c = C[q],
 * S = sum((w - mu)(c - mean c)) / (sum((c - mean c)^2) + 1e-8), Z = mu - S mean(c).
 * Sums run left to right over the 32 weights.  scales = FP16(S), zeros = FP16(Z).
 * Errors as wq_quantize_w4. */
int wq_quantize_w2(const float* W, int64_t N, int64_t K, int32_t group,
                   uint8_t* codes, uint16_t* scales, uint16_t* zeros);

/* Packs FP16 W4 zero points [N][G] (as wq_quantize_w4 writes them) two per
 * byte (SPECTRA section 3.4): zeros_packed[n][m] = z[n][2m] | z[n][2m+1] << 4,
 * [N][ceil(G/2)].  Errors: WQ_ERR_INVALID_ARG for NULL pointers, bad N/K, or a
 * zero point that is not an integer in 0..15. */
int wq_pack_zeros_w4(const uint16_t* zeros, int64_t N, int64_t K, uint8_t* zeros_packed);

/* Profile-guided outlier selection (OTF-LLM v4.0 section 4):
 * score_c = sqrt(sum_n W[n][c]^2) * profile[c] (float64, rows summed in order);
 * n_out = floor(ratio * K); the n_out highest scores (ties to the lower index),
 * written ascending to idx (int32, SPECTRA section 3.3).  idx_cap is the
 * capacity of idx; *n_out receives the count.
 * Errors: WQ_ERR_INVALID_ARG if ratio is outside [0, 1], idx_cap < n_out, or a
 * pointer is NULL. */
int wq_select_outliers(const float* W, int64_t N, int64_t K, const double* profile,
                       double ratio, int32_t* idx, int64_t idx_cap, int64_t* n_out);

/* Kurtosis-adaptive outlier selection (SPECTRA sections 3.1-3.3), a host
 * policy that picks n_out itself:
 *   saliency S_c = |gamma_c| * sqrt(sum_n W[n][c]^2)  (float64, rows in order;
 *                  gamma NULL means gamma_c = 1, the page's fallback for
 *                  projections with no preceding normalization gain);
 *   kappa = population kurtosis of S (mean, variance and fourth moment summed
 *           left to right; 0 when all S are equal);
 *   r = clamp(r_base * (1 + 0.15 * log1p(max(0, kappa - 3))), 0.005, 0.03);
 *   n_out = floor(r * K) columns of highest S (ties to the lower index), written
 *           ascending to idx.
 * r_base is 0.01 on the page.  idx_cap >= floor(0.03 K) always suffices.
 * *ratio and *kappa receive r and kappa (either may be NULL).
 * Errors: WQ_ERR_INVALID_ARG for NULL W / n_out, r_base outside (0, 1], or a
 * short idx. */
int wq_select_outliers_kurtosis(const float* W, int64_t N, int64_t K, const double* gamma,
                                double r_base, int32_t* idx, int64_t idx_cap, int64_t* n_out,
                                double* ratio, double* kappa);

/* Outlier split (SPECTRA section 3.4 "dense residual"; section 3.6 payload):
 * W_dense = W with columns idx[] set to 0 (W_dense may alias W), and
 * W_out[n][j] = FP16(W[n][idx[j]]) (round to nearest even).
 * Errors: WQ_ERR_INVALID_ARG if idx is not strictly increasing within [0, K). */
int wq_split_outliers(const float* W, int64_t N, int64_t K, const int32_t* idx,
                      int64_t n_out, float* W_dense, uint16_t* W_out);

/* Dequantize on the host to FP16 [N][K]:
 * W4, W4P  w_hat = FP16((q - z) * s)            (the float32 product is exact)
 * W2       w_hat = FP16(float32(S * C[q] + Z))  (one float32 rounding, then FP16).
 * fmt is WQ_FMT_W4, WQ_FMT_W4P or WQ_FMT_W2. */
int wq_dequant_host(int fmt, const uint8_t* codes, const uint16_t* scales,
                    const uint16_t* zeros, int64_t N, int64_t K, uint16_t* W_hat);

/* Refinement columns of a packed layer (StrataFlux page, section 3.2.1: the
 * weight residual, stored as 4-bit integers with their own scale factors):
 *   R = W - w_hat  in float32 (w_hat the FP16 dequantized layer, as
 *       wq_dequant_host makes it), with R[:, c] = 0 for every outlier column c
 *       in out_idx (the resident layer holds those exactly in FP16);
 *   R^T [K][N] quantized in the W4 format along N (wq_quantize_w4 of R^T:
 *       groups of 32 output rows): rcodes [K][N/2], rscales, rzeros [K][N/32].
 * W is the float32 layer [N][K] before the outlier split; codes / scales /
 * zeros its packed form in fmt (WQ_FMT_W4, WQ_FMT_W4P or WQ_FMT_W2); out_idx
 * int32 [n_out] strictly increasing in [0, K) (NULL when n_out == 0).  These
 * are the columns wq_refine_add, wq_refine_topk and wq_gemv_tiled_refine add.
 * Works on 32 output rows at a time (host memory of about 200 K bytes).
 * Errors: WQ_ERR_UNSUPPORTED unless N % 32 == 0 and N <= 65536;
 * WQ_ERR_INVALID_ARG for NULL pointers, bad shapes or indices. */
int wq_refinement_w4(int fmt, const float* W, const uint8_t* codes, const uint16_t* scales,
                     const uint16_t* zeros, int64_t N, int64_t K, const int32_t* out_idx,
                     int64_t n_out, uint8_t* rcodes, uint16_t* rscales, uint16_t* rzeros);

/* ------------------------------------------------------------- device (HIP)
 * All device pointers; `stream` is a hipStream_t (NULL = null stream).
 */

/* Device dequantize, bit-identical to wq_dequant_host.  The unfused two-kernel
 * baseline that SPECTRA section 4.1 argues against (dequantize to memory, then
 * multiply) is built from this. */
int wq_dequant_device(int fmt, const uint8_t* codes, const uint16_t* scales,
                      const uint16_t* zeros, int64_t N, int64_t K, uint16_t* W_hat,
                      void* stream);

/* Fused M = 1 W4 GEMV (SPECTRA section 4.1):
 *   y[n] = FP16( sum_{k not in out_idx} w_hat[n][k] x[k]
 *                + sum_j out_w[n][j] x[out_idx[j]] )      with FP32 accumulation.
 * With flags & WQ_FUSE_OUTLIERS the outlier sum is added in the same launch;
 * without it the background still skips out_idx and the caller adds the
 * outliers with wq_outlier_add.  n_out == 0 means no outliers (out_idx and
 * out_w may be NULL).  x and y must not overlap. */
int wq_gemv_w4(const uint8_t* codes, const uint16_t* scales, const uint16_t* zeros,
               int64_t N, int64_t K, const int32_t* out_idx, const uint16_t* out_w,
               int64_t n_out, uint32_t flags, const uint16_t* x, uint16_t* y,
               void* stream);

/* Fused M = 1 W2 GEMV (OTF-LLM v4.0 section 5 and "continuous GEMM addition"),
 * same contract as wq_gemv_w4 with w_hat = S * C[q] + Z. */
int wq_gemv_w2(const uint8_t* codes, const uint16_t* scales, const uint16_t* zeros,
               int64_t N, int64_t K, const int32_t* out_idx, const uint16_t* out_w,
               int64_t n_out, uint32_t flags, const uint16_t* x, uint16_t* y,
               void* stream);

/* Fused M = 1 GEMV of a W4P layer: wq_gemv_w4 with the zero points read from
 * their packed bytes ([N][ceil(G/2)], layout above); identical results. */
int wq_gemv_w4p(const uint8_t* codes, const uint16_t* scales, const uint8_t* zeros_packed,
                int64_t N, int64_t K, const int32_t* out_idx, const uint16_t* out_w,
                int64_t n_out, uint32_t flags, const uint16_t* x, uint16_t* y,
                void* stream);

/* Small-M batched product on matrix cores (SPECTRA section 4.2; M is a
 * runtime argument): Y[m][n] = FP16(sum_k X[m][k] w_hat[n][k] + outliers) for
 * 1 <= M <= WQ_GEMM_MAX_M, fmt WQ_FMT_W4, WQ_FMT_W4P or WQ_FMT_W2.  X is [M][K], Y is [M][N].
 * M > WQ_GEMM_MAX_M returns WQ_ERR_UNSUPPORTED. */
int wq_gemm_wq(int fmt, const uint8_t* codes, const uint16_t* scales, const uint16_t* zeros,
               int64_t N, int64_t K, const int32_t* out_idx, const uint16_t* out_w,
               int64_t n_out, uint32_t flags, const uint16_t* X, int64_t M, uint16_t* Y,
               void* stream);

/* Embedding row gather (SPECTRA section 4.3): out[t][k] = w_hat[ids[t]][k] for
 * t < n_ids, FP16 [n_ids][K], bit-identical to wq_dequant_device of those rows
 * (W4 / W4P / W2 table [V][K] in the layouts above; ids int32 on the device).
 * Only the rows named by ids are read.  An id outside [0, V) yields a row of
 * zeros (the ids are not checked on the host).  n_ids == 0 does nothing. */
int wq_embed_gather(int fmt, const uint8_t* codes, const uint16_t* scales, const uint16_t* zeros,
                    int64_t V, int64_t K, const int32_t* ids, int64_t n_ids, uint16_t* out,
                    void* stream);

/* ------------------------------------------- runtime top-k refinement
 * StrataFlux page, section 3.2.1: channel selection per chunk of input channels
 * and the refinement add of Eq. 2.  The refinement columns C are given per
 * input channel, i.e. C transposed [K][N], in the W4 format along N (codes
 * [K][N/2], FP16 scales and zeros [K][N/32], groups of 32 output rows); the
 * plain reading is the 4-bit residual W - w_hat of the resident layer. */

/* Number of channels wq_topk_chunks selects: per full chunk min(k, chunk), and
 * min(k, K % chunk) for a short last chunk.  Negative WQ_ERR_* on bad sizes. */
int64_t wq_topk_count(int64_t K, int64_t chunk, int64_t k);

/* S(x): in each chunk of `chunk` consecutive channels of x (FP16 [K]), the k
 * channels of largest |x| (ties to the lower index), exact.  Chunk c's picks are
 * written ascending to sel[c * min(k, chunk) ...]; sel (int32, device) holds
 * wq_topk_count(K, chunk, k) entries.  chunk: a multiple of 64 in [64, 1024]
 * (the page uses 1024).  K % 32 == 0.  k == 0 does nothing. */
int wq_topk_chunks(const uint16_t* x, int64_t K, int64_t chunk, int64_t k, int32_t* sel,
                   void* stream);

/* Eq. 2: y[n] = FP16( y[n] + sum_j x[sel[j]] C[n][sel[j]] ), FP32 accumulation,
 * j < n_sel, with C[n][i] = (q - z) s of the W4 refinement row i (values as
 * dequantized, without their FP16 rounding).  Entries of sel outside [0, K)
 * are skipped.  N % 32 == 0.  y is read and written in place. */
int wq_refine_add(const uint8_t* rcodes, const uint16_t* rscales, const uint16_t* rzeros,
                  int64_t N, int64_t K, const int32_t* sel, int64_t n_sel, const uint16_t* x,
                  uint16_t* y, void* stream);

/* Selection and add in one launch: y += sum over S(x) of x_i C[:, i], with S(x)
 * exactly as wq_topk_chunks makes it, and the sums in the same order as
 * wq_topk_chunks followed by wq_refine_add (the two give identical y).  Every
 * workgroup selects for itself from x, so the selection never goes through
 * global memory; sel_out (int32, device, wq_topk_count(K, chunk, k) entries)
 * receives S(x) if not NULL.  With sel_out given and more than 8 chunks (or
 * more than 4096 selected channels), the call runs wq_topk_chunks then
 * wq_refine_add instead (faster there; the same y).  Without sel_out, more
 * than 4096 selected channels return WQ_ERR_UNSUPPORTED.  N % 32 == 0,
 * chunk a multiple of 64 in [64, 1024], x 16-byte aligned; k == 0 does
 * nothing. */
int wq_refine_topk(const uint8_t* rcodes, const uint16_t* rscales, const uint16_t* rzeros,
                   int64_t N, int64_t K, int64_t chunk, int64_t k, const uint16_t* x, uint16_t* y,
                   int32_t* sel_out, void* stream);

/* Standalone outlier correction (the add of SPECTRA section 4.1's outlier loop;
 * the same arithmetic as the column refinement add of the StrataFlux page,
 * section 3.2.1 Eq. 2, for a static column set):
 *   Y[m][n] = FP16( Y[m][n] + sum_j out_w[n][j] X[m][idx[j]] ),  FP32 accumulation.
 * Y is read and written in place. */
int wq_outlier_add(const int32_t* idx, const uint16_t* out_w, int64_t n_out, int64_t N,
                   const uint16_t* X, int64_t M, int64_t K, uint16_t* Y, void* stream);

/* ------------------------------------------------------ tiled M = 1 layout
 * A second device layout of the same packed layer, read by the matrix-core
 * M = 1 kernel so that every 64-lane load is one contiguous 1 KB block (the
 * row-major arrays above make each load touch 16 rows).  It holds the bytes of
 * codes / scales / zeros / out_w, rearranged and zero-padded; the outlier
 * indices stay a separate int32 array.  SPECTRA section 3.4 names an
 * interleaved, hardware-tiled layout for its kernel; this is the gfx950 one.
 *
 * Geometry: nrb = ceil(N / 16) row blocks, nks = ceil(K / 512) slices,
 * nch = ceil(n_out / 8) outlier chunks, SB = 256 (W4) or 128 (W2) code bytes
 * per row and slice.  Three sections, each starting at a multiple of 256 bytes
 * (codes at 0, then meta, then slab); every entry past N, K or n_out is 0.
 *   codes: tile (b, s) of 16 SB bytes at (b nks + s) 16 SB; its byte
 *          1024 u + 16 (n + 16 r) + c   (u < SB / 64, n < 16, r < 4, c < 16)
 *          = codes[16 b + n][s SB + 64 u + 16 r + c]
 *   meta:  tile (b, s) of 512 FP16 entries at (b nks + s) 1024 bytes; entry
 *          8 (n + 16 r) + i     = scales[16 b + n][16 s + 4 r + i]  (i < 4)
 *          8 (n + 16 r) + 4 + i = zeros [16 b + n][16 s + 4 r + i]
 *          W4P: tile (b, s) of 640 bytes at (b nks + s) 640; FP16 entry
 *          4 (n + 16 r) + i = scales[16 b + n][16 s + 4 r + i], and bytes
 *          512 + 2 (n + 16 r) + j (j < 2) = zeros_packed[16 b + n][8 s + 2 r + j]
 *   slab:  chunk (b, c) of 128 FP16 entries at (b nch + c) 256 bytes; entry
 *          8 n + i = out_w[16 b + n][8 c + i]                       (i < 8)
 */

/* Bytes of the tiled layout of an N x K layer with n_out outlier columns, or a
 * negative WQ_ERR_* code for invalid arguments (fmt, shape as above). */
int64_t wq_tiled_bytes(int fmt, int64_t N, int64_t K, int64_t n_out);

/* Host rearrangement of row-major packed arrays (layouts above; out_w may be
 * NULL when n_out == 0) into the tiled layout.  `tiled` holds `tiled_bytes`
 * bytes, at least wq_tiled_bytes(...); every byte of the layout is written.
 * Errors: WQ_ERR_INVALID_ARG for NULL pointers, bad shapes or a short buffer. */
int wq_tile_host(int fmt, const uint8_t* codes, const uint16_t* scales, const uint16_t* zeros,
                 const uint16_t* out_w, int64_t N, int64_t K, int64_t n_out, uint8_t* tiled,
                 int64_t tiled_bytes);

/* Fused M = 1 GEMV on a tiled layer (device pointer `tiled`), outliers always
 * in the same launch; the same result contract as wq_gemv_w4 / wq_gemv_w2
 * with WQ_FUSE_OUTLIERS.  WQ_ERR_UNSUPPORTED for shapes the kernel cannot hold:
 * K > 32768, more than 32 outlier positions per 512-channel slice
 * (n_out > 32 ceil(K / 512)), or partial sums beyond the 160 KB of LDS
 * (N above about 200 000 rows at K = 32768). */
int wq_gemv_tiled(int fmt, const uint8_t* tiled, int64_t N, int64_t K, const int32_t* out_idx,
                  int64_t n_out, const uint16_t* x, uint16_t* y, void* stream);

/* The tiled layer against M = 1 to WQ_GEMM_MAX_M activation rows: Y [M][N] =
 * X [M][K] times the layer (outlier pass fused), the batched product of
 * SPECTRA section 4.2 (M a runtime argument).  Up to 4 rows (W2: 2) share the
 * matrix-core kernel's 16 group slots (each 512-channel slice taken in M
 * windows of 16 / M groups; 3 rows run as 4), so the codes are decoded once
 * for all rows; past that, or where the slot kernel does not fit, the batched
 * kernel reads the same tiles (each wave load four contiguous 256-byte runs),
 * dequantizes them to FP16 and multiplies them with the M rows on the matrix
 * cores.  M = 1 is wq_gemv_tiled.  Limits: those of wq_gemv_tiled, and for
 * M > 1 on the batched kernel at most 1024 outlier columns and its partial
 * sums within the LDS; other shapes return WQ_ERR_UNSUPPORTED (wq_gemm_wq on
 * the row-major arrays takes every M up to 16). */
int wq_gemm_tiled(int fmt, const uint8_t* tiled, int64_t N, int64_t K, const int32_t* out_idx,
                  int64_t n_out, const uint16_t* X, int64_t M, uint16_t* Y, void* stream);

/* The tiled M = 1 product with the runtime top-k refinement of StrataFlux
 * (section 3.2.1, Eq. 2) in the same launch:
 *   y[n] = FP16( sum_k w_hat[n][k] x[k] (outlier pass fused)
 *                + sum_{i in S(x)} x_i C[n][i] ),   FP32 accumulation,
 * with S(x) exactly as wq_topk_chunks makes it and C the W4 refinement columns
 * of wq_refine_add (rcodes [K][N/2], rscales / rzeros [K][N/32]).  Every
 * workgroup selects for itself while its first weights are in flight, loads
 * the picked columns for its own row blocks behind them, and adds their
 * products before the one rounding to FP16.  sel_out (int32, device,
 * wq_topk_count(K, chunk, k) entries) receives S(x) if not NULL.  Where the
 * one-launch kernel does not fit (more than 4 units of one chunk, 32 picks
 * and one row block per lane, i.e. large k, many chunks per wave or many row
 * blocks per workgroup; or LDS), the call runs wq_gemv_tiled and then
 * wq_refine_topk: the same selection, and y within the same bound, but with
 * the product rounded to FP16 before the add.  Limits: those of
 * wq_gemv_tiled, plus N % 32 == 0, chunk a multiple of 64 in [64, 1024], and
 * rcodes, x, y 16-byte aligned; k == 0 is wq_gemv_tiled alone. */
int wq_gemv_tiled_refine(int fmt, const uint8_t* tiled, int64_t N, int64_t K,
                         const int32_t* out_idx, int64_t n_out, const uint16_t* x, uint16_t* y,
                         const uint8_t* rcodes, const uint16_t* rscales, const uint16_t* rzeros,
                         int64_t chunk, int64_t k, int32_t* sel_out, void* stream);

/* ------------------------------------------------ kernel-variant selection
 * Not part of the method: for tests and measurements that run a call on each
 * of the kernels the library could choose for it.  Each *_v entry point is
 * the entry point of the same name without the suffix, with an explicit
 * choice of kernel; NULL (or a field < 0) keeps the library's own choice,
 * which is what the plain entry points use.  Every variant meets the same
 * result contract (bit-identical results where the plain entry point's
 * comment says so, else within the same bound).  Nothing is remembered
 * between calls. */
typedef struct wq_variant {
  /* M = 1 GEMV on the row-major arrays: 0 the VALU kernels, 1 the library's
   * rule, 2 the matrix-core kernel wherever it takes the shape */
  int32_t gemv_kernel;
  /* VALU GEMV: rows per wave step (1..4), and 0 / 1 to keep x in registers /
   * stage it in LDS (where the LDS fits) */
  int32_t gemv_rows_per_wave;
  int32_t gemv_lds_x;
  /* wq_gemm_wq at 2 <= M: 0 the per-group tile kernel only, 1 the rule, 2 the
   * persistent matrix-core kernels wherever they take the shape; gemm_rows 0
   * skips the shared-slot kernel of M <= 4 (wq_gemm_wq and wq_gemm_tiled) */
  int32_t gemm_kernel;
  int32_t gemm_rows;
  /* persistent batched kernel: groups per lane quarter of a slice (2 or 4;
   * layers without outliers), and 0 / 1 to load the activation rows in the
   * lane layout / whole through an LDS transpose (where the LDS fits) */
  int32_t batch_slice_groups;
  int32_t batch_row_transpose;
  /* refinement add: 1, 2 or 4 groups of 32 output rows per workgroup */
  int32_t refine_groups;
  /* wq_gemv_tiled_refine: 0 runs the product and then wq_refine_topk (two
   * launches); refine_wide 0 keeps the one-launch kernel at 12 waves where
   * the library would take 16 */
  int32_t refine_fuse;
  int32_t refine_wide;
  /* persistent batched kernel: 0 keeps each wave's partial tiles in LDS, 1
   * in registers wherever a workgroup has at most 8 row blocks (the same
   * bits); the library's choice takes registers only where that leaves room
   * for the staged activation rows */
  int32_t batch_register_partials;
} wq_variant;

int wq_gemv_v(int fmt, const uint8_t* codes, const uint16_t* scales, const uint16_t* zeros,
              int64_t N, int64_t K, const int32_t* out_idx, const uint16_t* out_w, int64_t n_out,
              uint32_t flags, const uint16_t* x, uint16_t* y, const wq_variant* variant,
              void* stream);
int wq_gemm_wq_v(int fmt, const uint8_t* codes, const uint16_t* scales, const uint16_t* zeros,
                 int64_t N, int64_t K, const int32_t* out_idx, const uint16_t* out_w,
                 int64_t n_out, uint32_t flags, const uint16_t* X, int64_t M, uint16_t* Y,
                 const wq_variant* variant, void* stream);
int wq_gemm_tiled_v(int fmt, const uint8_t* tiled, int64_t N, int64_t K, const int32_t* out_idx,
                    int64_t n_out, const uint16_t* X, int64_t M, uint16_t* Y,
                    const wq_variant* variant, void* stream);
int wq_refine_add_v(const uint8_t* rcodes, const uint16_t* rscales, const uint16_t* rzeros,
                    int64_t N, int64_t K, const int32_t* sel, int64_t n_sel, const uint16_t* x,
                    uint16_t* y, const wq_variant* variant, void* stream);
int wq_refine_topk_v(const uint8_t* rcodes, const uint16_t* rscales, const uint16_t* rzeros,
                     int64_t N, int64_t K, int64_t chunk, int64_t k, const uint16_t* x,
                     uint16_t* y, int32_t* sel_out, const wq_variant* variant, void* stream);
int wq_gemv_tiled_refine_v(int fmt, const uint8_t* tiled, int64_t N, int64_t K,
                           const int32_t* out_idx, int64_t n_out, const uint16_t* x, uint16_t* y,
                           const uint8_t* rcodes, const uint16_t* rscales, const uint16_t* rzeros,
                           int64_t chunk, int64_t k, int32_t* sel_out, const wq_variant* variant,
                           void* stream);

/* -------------------------------------------------- measurement support
 * Not part of the method: kernels of known traffic that calibrate bandwidth
 * figures and hardware byte counters. */

/* Streams `bytes` (multiple of 16) from `src` and writes one uint32 per
 * workgroup to `sink` (sink must hold wq_read_probe_sink_words(bytes) words). */
int wq_read_probe(const void* src, int64_t bytes, uint32_t* sink, void* stream);
int64_t wq_read_probe_sink_words(int64_t bytes);

/* The same streaming read with a chosen launch geometry, for finding the
 * attainable rate at a given size: a grid-stride sweep by `blocks` workgroups
 * of `threads` threads (a multiple of 64, at most 1024), each thread with
 * `ring` 16-byte loads in flight per round (1, 2, 4, 8 or 16); blocks == 0
 * takes enough workgroups for one round (one-shot).  sink holds as many
 * uint32 words as workgroups (at most 65536).  bytes < 2 GB. */
int wq_read_probe_geom(const void* src, int64_t bytes, uint32_t* sink, int blocks, int threads,
                       int ring, void* stream);

/* Copies `bytes` (multiple of 16) from src to dst with 16-byte vector loads
 * and stores. */
int wq_copy_probe(const void* src, void* dst, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* WQ_H */
