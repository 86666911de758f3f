/*
 * moe_mi355x.h - C ABI of the MI355X (gfx950) routed-expert MoE forward and
 * fused SwiGLU + FP8 activation quantizer (libmoe_mi355x.so).
 *
 * Conventions for every entry point
 *   - Tensor pointers are device memory owned by the caller, contiguous and
 *     row-major; bf16 tensors are passed as uint16_t bit patterns. 16-byte
 *     vectorised tensors (bf16 activations and weights, FP8 outputs) must be
 *     16-byte aligned.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the default
 *     stream). No entry point synchronises the stream or the device, copies
 *     to or from the host, or allocates memory; scratch space, where needed,
 *     is a caller-provided workspace.
 *   - Return value: MOE_OK, or a negative code. On MOE_ERR_INVALID_ARG and
 *     MOE_ERR_UNSUPPORTED nothing has been enqueued and outputs are untouched.
 *     moe_last_error() gives a message for the calling thread's last failure.
 *   - Empty work (T = 0 or M = 0) returns MOE_OK and enqueues nothing unless
 *     the entry point says otherwise.
 *   - Results are deterministic: the same inputs give the same bytes, run to
 *     run (no atomics whose order reaches an output).
 *   - Calls that evaluate the SwiGLU (swiglu, swiglu_quant_fp8, tile_quant_fp8
 *     with swiglu = 1, and the fused gate_up GEMMs on their 256-row path)
 *     first enqueue a small kernel on `stream` that writes a constant table
 *     of exact SiLU values into a file-scope device array of the library
 *     (static storage, not an allocation); concurrent calls on other streams
 *     write the same bits into it.
 *
 * Page citations name the five source pages by title:
 *   TileOPs #778  "[Feat][MoE] SharedFusedMoE with native shared expert kernel and TP support"
 *   TileOPs #1580 "[Perf][MoE] Grouped-GEMM TMA OOB zero-fill + unpermute out=: ..."
 *   pypto-lib #809 "perf(dsv4/moe): predicate empty routed-expert stages"
 *   TileLang tutorial Example 07 "MoE dispatch contract and quantized GEMM"
 *   xtuner #2089 "[Feat] Fuse MoE activation FP8 quantization kernels"
 */
#ifndef MOE_MI355X_H_
#define MOE_MI355X_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK 0
#define MOE_ERR_INVALID_ARG (-1) /* null pointer, bad shape, misalignment */
#define MOE_ERR_UNSUPPORTED (-2) /* valid but outside what the kernels handle */
#define MOE_ERR_HIP (-3)         /* a HIP launch reported an error */

/* Message for the calling thread's most recent failure ("" if none). */
const char* moe_last_error(void);

/* ABI revision of this header; bumps whenever a signature changes. */
int moe_abi_version(void);

/* Number of padded row blocks the grouped GEMMs iterate over, an upper bound
 * that depends only on host-known sizes:
 *     ceil(numel / block_m) + E * (padding_m / block_m).
 * Tutorial Example 07, expected output: 18 pairs, 4 experts, 128-row blocks
 * and padding give 5 = ceil(18/128) + 4. The page always has padding_m ==
 * block_m; a larger multiple lets each expert's padding span that many
 * blocks. Returns -1 for non-positive block_m / padding_m or padding_m not a
 * multiple of block_m. Host-only, no device work. */
int64_t moe_num_blocks(int64_t numel, int E, int block_m, int padding_m);

/* Bytes of device workspace moe_align needs for numel = T*top_k pairs over E
 * experts. */
size_t moe_align_workspace_bytes(int64_t numel, int E);

/* Scoring functions of moe_topk_softmax. */
#define MOE_SCORING_SOFTMAX 0 /* softmax over all E experts (the workloads of TileOPs #1580) */
#define MOE_SCORING_SIGMOID 1 /* logistic sigmoid per expert ("sigmoid routing", the Kimi-K2
                                 benchmark of TileOPs #778) */

/* Top-k routing.
 * logits       [T, E] float32 router scores ("gating", TileOPs #778,
 *              "Partial output contract").
 * expert_bias  [E] float32 or NULL: added to every row of logits (one fp32
 *              addition) before selection and scoring.
 * scoring      MOE_SCORING_SOFTMAX or MOE_SCORING_SIGMOID.
 * renormalize  1: weights are the selected experts' scores divided by their
 *              sum (for softmax: a softmax over the selected logits), so each
 *              row sums to 1; 0: the scores themselves (softmax probability
 *              over all E, or the sigmoid).
 * topk_ids     [T, top_k] int32 out: experts in descending order of
 *              logit + bias; equal values go to the lower expert id.
 * topk_weights [T, top_k] float32 out, slot order as topk_ids.
 * Limits: 1 <= E <= 1024, 1 <= top_k <= min(E, 16). Non-finite logits are
 * not supported. Returns MOE_ERR_INVALID_ARG for another scoring or
 * renormalize value. */
int moe_topk_softmax(const float* logits, const float* expert_bias, int64_t T, int E, int top_k, int scoring,
                     int renormalize, int32_t* topk_ids, float* topk_weights, hipStream_t stream);

/* Dispatch tables of Tutorial Example 07 ("moe_dispatch_contract.py": the
 * four host-side tables and the kernel-side row recovery), built on the
 * device with wavefront ballots and prefix scans; no host synchronisation.
 * topk_ids             [T, top_k] int32 in, each in [0, E).
 * group_sizes          [E] out: pairs routed to each expert.
 * group_offsets        [E] out: exclusive prefix sum of group_sizes (start of
 *                      each expert's rows in the compact layout).
 * group_padded_offsets [E] out: exclusive prefix sum of the sizes rounded up
 *                      to padding_m (an empty expert pads to 0 rows).
 * group_idx_for_bx     [moe_num_blocks(T*top_k, E, block_m, padding_m)] out:
 *                      expert owning padded row block bx = the last expert
 *                      whose padded offset is <= bx*block_m.
 * sorted_pair          [T*top_k] out: pair index p = t*top_k + j of compact
 *                      row r; rows of one expert keep ascending p.
 * pair_to_row          [T*top_k] out: inverse permutation of sorted_pair.
 * workspace            >= moe_align_workspace_bytes(T*top_k, E) bytes.
 * Requires padding_m % block_m == 0, 1 <= E <= 1024, T*top_k < 2^31.
 * With T = 0 the E-sized tables and group_idx_for_bx are still written. */
int moe_align(const int32_t* topk_ids, int64_t T, int top_k, int E, int padding_m, int block_m,
              int32_t* group_sizes, int32_t* group_offsets, int32_t* group_padded_offsets,
              int32_t* group_idx_for_bx, int32_t* sorted_pair, int32_t* pair_to_row,
              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* moe_align for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same tables, bytes and launches as moe_align, with the chunk histogram in
 * a static per-device array of the library (moe_align_noalloc_max_scratch_bytes()
 * bytes, 4 MiB, held on each GPU the library runs on until the process
 * ends) instead of a caller workspace. It calls no allocating routine; its
 * first call on a device looks up that device's copy of the array
 * (hipGetSymbolAddress). Every call on one GPU shares the array: calls that
 * overlap on one GPU (two streams, two threads) race and give wrong tables.
 * The stream must belong to the current device (MOE_ERR_INVALID_ARG
 * otherwise). Pair counts whose histogram, moe_align_workspace_bytes(T*top_k,
 * E), exceeds the array are refused with MOE_ERR_UNSUPPORTED before anything
 * is enqueued (at E = 256 up to 4,194,304 pairs). Other limits and errors as
 * moe_align. */
int moe_align_noalloc(const int32_t* topk_ids, int64_t T, int top_k, int E, int padding_m, int block_m,
                      int32_t* group_sizes, int32_t* group_offsets, int32_t* group_padded_offsets,
                      int32_t* group_idx_for_bx, int32_t* sorted_pair, int32_t* pair_to_row, hipStream_t stream);

/* Size in bytes of moe_align_noalloc's static scratch array. */
size_t moe_align_noalloc_max_scratch_bytes(void);

/* Token permute into the compact expert-major layout (TileOPs "MoePermuteAlignOp":
 * token routing for the grouped GEMM):
 *     x_perm[r, :] = hidden[sorted_pair[r] / top_k, :]
 * equivalently x_perm[pair_to_row[p], :] = hidden[p / top_k, :].
 * hidden [T, H] bf16, x_perm [T*top_k, H] bf16. H % 8 == 0.
 * sorted_pair, pair_to_row: the two permutation tables of moe_align; either
 * may be NULL (not both). With pair_to_row (and top_k <= 16) the copy runs
 * token by token, reading each hidden row once; otherwise it gathers by
 * sorted_pair. Both give the same bytes. */
int moe_permute(const uint16_t* hidden, const int32_t* sorted_pair, const int32_t* pair_to_row, int64_t T,
                int top_k, int H, uint16_t* x_perm, hipStream_t stream);

/* Grouped GEMM for gate+up, C[e] = A[e] @ W[e]^T (TileOPs #1580, "Benchmark
 * results" and "Grouped-GEMM kernel"): A is the compact [numel, H] layout;
 * each expert's last, partial row block is masked inside the kernel (rows
 * past the expert are read from its last row and their outputs are never
 * stored) instead of padding A. Row blocks are decoded from the tables as in Tutorial Example 07:
 *     m_start = bx*block_m - group_padded_offsets[g] + group_offsets[g].
 * w_gate_up [E, 2F, H] bf16: rows 0..F-1 gate, rows F..2F-1 up.
 * fuse_swiglu = 0: out [numel, 2F] bf16 = bf16(A @ W^T).
 * fuse_swiglu = 1: out [numel, F] bf16 = bf16(silu(g) * u), g and u the bf16
 *   roundings of the gate and up products: byte-identical to the unfused
 *   GEMM followed by swiglu().
 * Tables are the moe_align outputs for the same (numel, E, padding_m,
 * block_m). Passing group_sizes = NULL (and the other three tables NULL)
 * treats A as one dense group of numel rows with E = 1 (the shared expert,
 * TileOPs #778 "SharedExpertMLPKernel").
 * Limits: block_m in {64, 128}; H % 64 == 0; F % 64 == 0; numel < 2^31.
 * Streams: some shapes run a persistent kernel (a fixed grid that claims its
 * tiles from device counters); each stream has its own counters (the first
 * 64 streams used; later streams, and hipStreamPerThread, take the kernel
 * with one workgroup per tile), and launches on one stream run in order. So
 * calls on different streams may overlap, but one graph captured from these
 * calls must not be replayed on two streams at the same time, nor replayed
 * while a call on its capture stream runs (the same holds for
 * grouped_gemm_gate_up_gather and grouped_gemm_down). */
int grouped_gemm_gate_up(const uint16_t* x_perm, const uint16_t* w_gate_up,
                         const int32_t* group_sizes, const int32_t* group_offsets,
                         const int32_t* group_padded_offsets, const int32_t* group_idx_for_bx,
                         int64_t numel, int E, int H, int F, int padding_m, int block_m,
                         int fuse_swiglu, uint16_t* out, hipStream_t stream);

/* grouped_gemm_gate_up with the token permute folded into its A loads: the
 * product of moe_permute followed by grouped_gemm_gate_up on x_perm (the
 * same bytes while T*H*2 < 2^32; past that this call takes the 128-row
 * kernel, whose fp32 sums may round differently), with compact row r of A
 * read from
 *     hidden[sorted_pair[r] / top_k, :]
 * (the permute's definition, TileOPs "MoePermuteAlignOp"; the grouped GEMM
 * of TileOPs #1580 "Grouped-GEMM kernel" on the permuted rows), so x_perm is
 * never written or read. hidden [T, H] bf16 (16-byte aligned),
 * sorted_pair [T*top_k] int32 from moe_align (values in [0, T*top_k); not
 * checked on the device), numel == T*top_k, the four tables non-NULL (no
 * dense mode). w_gate_up, fuse_swiglu, out, limits: as grouped_gemm_gate_up.
 * Returns MOE_ERR_INVALID_ARG for a NULL table or sorted_pair, or
 * numel != T*top_k. */
int grouped_gemm_gate_up_gather(const uint16_t* hidden, int64_t T, const int32_t* sorted_pair, int top_k,
                                const uint16_t* w_gate_up, const int32_t* group_sizes,
                                const int32_t* group_offsets, const int32_t* group_padded_offsets,
                                const int32_t* group_idx_for_bx, int64_t numel, int E, int H, int F,
                                int padding_m, int block_m, int fuse_swiglu, uint16_t* out,
                                hipStream_t stream);

/* SwiGLU on the gate|up halves: h[m, f] = bf16(silu(gate[m, f]) * up[m, f])
 * with gate = gate_up[:, 0:F], up = gate_up[:, F:2F] (TileOPs #778 "SiLU-mul";
 * xtuner #2089 native_swiglu). silu uses the library's fp32 exp sequence
 * (moe_common.h). gate_up [M, 2F] bf16, h [M, F] bf16, F % 8 == 0. */
int swiglu(const uint16_t* gate_up, int64_t M, int F, uint16_t* h, hipStream_t stream);

/* Grouped GEMM for down, y[e] = h[e] @ W_down[e]^T, same masking and table
 * contract as grouped_gemm_gate_up. h [numel, F] bf16, w_down [E, H, F] bf16,
 * y [numel, H] bf16. NULL tables: one dense group (shared expert).
 * Limits: block_m in {64, 128}; F % 64 == 0; H % 128 == 0. */
int grouped_gemm_down(const uint16_t* h, const uint16_t* w_down, const int32_t* group_sizes,
                      const int32_t* group_offsets, const int32_t* group_padded_offsets,
                      const int32_t* group_idx_for_bx, int64_t numel, int E, int H, int F,
                      int padding_m, int block_m, uint16_t* y, hipStream_t stream);

/* Unpermute: weighted sum over each token's k expert outputs with
 * routed_scaling_factor applied before the single cast and store (TileOPs
 * #1580, "Unpermute"), plus an optional addend (the shared expert's output,
 * TileOPs #778 "Partial output contract") joined before that rounding:
 *     out[t] = bf16(rsf * sum_j topk_weights[t,j] * y[pair_to_row[t*k+j]] + addend[t])
 * y [T*top_k, H] bf16, pair_to_row [T*top_k] int32, topk_weights [T, top_k]
 * float32, addend [T, H] bf16 or NULL, out [T, H] bf16 (may not alias y).
 * Sum in fp32, j ascending. H % 8 == 0, top_k <= 16. */
int moe_unpermute(const uint16_t* y, const int32_t* pair_to_row, const float* topk_weights,
                  int64_t T, int top_k, int H, float routed_scaling_factor,
                  const uint16_t* addend, uint16_t* out, hipStream_t stream);

/* Fused SwiGLU + FP8 quantizer (xtuner #2089, swiglu_per_tile_quant_with_
 * trans_per_block): h = swiglu(gate_up) is formed in registers, never stored,
 * and quantized to OCP e4m3 (max 448) in two layouts in one pass:
 *   row layout  q_row [M, F] uint8, s_row [M, F/128] float32: per 1x128 tile
 *               of a row, s = fl32(amax/448), code = e4m3(fl32(h/s));
 *   transposed  q_t [F, M_pad] uint8, s_t [F/128, M_pad/128] float32 with
 *               M_pad = ceil(M/128)*128: per 128x128 block (amax over real
 *               rows), q_t[f, m] = e4m3(fl32(h[m, f]/s)); pad columns 0x00.
 * Divisions are correctly rounded fp32, e4m3 rounding is nearest-even; a tile
 * with amax 0 has scale 0 and codes 0x00. The bytes equal swiglu() followed
 * by the two quantizers. gate_up [M, 2F] bf16; F % 128 == 0; M < 2^31. */
int swiglu_quant_fp8(const uint16_t* gate_up, int64_t M, int F, uint8_t* q_row, float* s_row,
                     uint8_t* q_t, float* s_t, hipStream_t stream);

/* The 1x128-tile FP8 quantizer family of xtuner #2089 ("Changes":
 * per_tile_quant_with_trans_per_block, per_tile_quant_with_trans_per_tile,
 * and with swiglu=1 swiglu_per_tile_quant_with_trans_per_block), on rows
 * grouped by expert with the "expand_128x" transposed layout.
 *   x            swiglu=0: the bf16 activation [M, K]; swiglu=1: gate_up
 *                [M, 2K] (gate columns first), quantizing h = swiglu(x) [M, K]
 *                exactly as swiglu_quant_fp8 does.
 *   group_sizes  device int32 [E], consecutive row ranges summing to M, or
 *                NULL for one group of M rows (E is then ignored).
 *   m_pad        width of q_t: a multiple of 128 no smaller than the groups'
 *                padded total sum(ceil(group_sizes[e]/128)*128) (with NULL
 *                groups, ceil(M/128)*128); tile_quant_fp8_m_pad_bound(M, E)
 *                always suffices. With grouped rows the kernel cannot check
 *                it: a group past m_pad gets no outputs at all.
 *   row layout   q_row [M, K] uint8, s_row [M, K/128] float32, per 1x128 tile
 *                of a row (as swiglu_quant_fp8).
 *   transposed   q_t [K, m_pad] uint8: group e's rows fill ceil(gs/128)*128
 *                columns starting at the previous groups' padded total; pad
 *                columns and columns past the total are 0x00.
 *                per_tile=0: s_t [K/128, m_pad/128], one scale per 128x128
 *                block of a group (amax over real rows);
 *                per_tile=1: s_t [K, m_pad/128], one scale per column and
 *                128-row tile of a group. Scales past the total are 0.
 *   q_t = s_t = NULL: the row layout only (what a forward GEMM on the
 *                codes reads); group_sizes, E, per_tile and m_pad then play
 *                no part, and the row bytes are those of the full call.
 * Scales fl32(amax/448), codes e4m3(fl32(h/s)), zero tiles 0x00 as above.
 * Rows must be 16-byte aligned (x, q_row, q_t); K % 128 == 0; M, m_pad < 2^31.
 * Returns MOE_ERR_INVALID_ARG for bad sizes or flags, or for exactly one of
 * q_t, s_t NULL (nothing enqueued); M = 0 with m_pad > 0 zero-fills q_t and
 * s_t. */
int tile_quant_fp8(const uint16_t* x, int64_t M, int K, int swiglu, const int32_t* group_sizes, int E,
                   int per_tile, int64_t m_pad, uint8_t* q_row, float* s_row, uint8_t* q_t, float* s_t,
                   hipStream_t stream);

/* 128 * (ceil(M/128) + E): a q_t width that covers any grouping of M rows into
 * E groups (host-only; -1 for negative arguments). */
int64_t tile_quant_fp8_m_pad_bound(int64_t M, int E);

/* Weight preparation for grouped_gemm_fp8: e4m3 codes of a bf16 weight matrix
 * w [rows, K] (for expert weights, rows = E*N) with one scale per 128x128
 * block, in the weight's own row-major layout: q [rows, K] uint8, s [rows/128,
 * K/128] float32, s = fl32(amax/448), code = e4m3(fl32(w/s)), an all-zero
 * block has scale 0 and codes 0x00. rows and K multiples of 128; w and q
 * 16-byte aligned. */
int fp8_block_quant_weights(const uint16_t* w, int64_t rows, int K, uint8_t* q, float* s, hipStream_t stream);

/* Block-scaled FP8 grouped GEMM, C[e] = A[e] @ W[e]^T on e4m3 operands (the
 * MoE path's down projection fed by the FP8 quantizer, xtuner #2089 "Summary":
 * W2 input quantization). A: codes qa [numel, K] with one scale per row and
 * 128-column tile sa [numel, K/128] (tile_quant_fp8's row layout); W: codes
 * qw [E, N, K] with one scale per 128x128 block sw [E, N/128, K/128]
 * (fp8_block_quant_weights). y [numel, N] bf16 = the fp32-accumulated sum of
 * the decoded products, each operand times its scale, rounded once. The four
 * dispatch tables as for grouped_gemm_down (all NULL: one dense group, E = 1).
 * N and K multiples of 128, block_m = 128, padding_m a multiple of 128;
 * qa, qw, y 16-byte aligned. MOE_ERR_UNSUPPORTED when numel * K or N * K
 * (the A codes, one group's weight codes) reach 2^32 bytes. */
int grouped_gemm_fp8(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                     const int32_t* group_sizes, const int32_t* group_offsets, const int32_t* group_padded_offsets,
                     const int32_t* group_idx_for_bx, int64_t numel, int E, int N, int K, int padding_m,
                     int block_m, uint16_t* y, hipStream_t stream);

/* The block-scaled FP8 grouped GEMM for gate+up: the product of
 * grouped_gemm_fp8 with w_gate_up's codes, optionally with SwiGLU fused into
 * its epilogue, and optionally reading the activation codes through the
 * dispatch permutation (as grouped_gemm_gate_up_gather does for bf16).
 *   qa, sa       e4m3 activation codes [a_rows, H] and their 1x128-tile
 *                scales [a_rows, H/128] (tile_quant_fp8's row layout).
 *                sorted_pair NULL: a_rows == numel, the compact permuted rows;
 *                otherwise a_rows == T with numel == T*top_k, and compact row
 *                r is row sorted_pair[r] / top_k (the token's codes, once per
 *                token instead of once per pair).
 *   qw, sw       fp8_block_quant_weights(w_gate_up): codes [E, 2F, H] (rows
 *                0..F-1 gate, F..2F-1 up), scales [E, 2F/128, H/128].
 *   fuse_swiglu  1: out [numel, F] bf16 = bf16(silu(g) * u) with g and u the
 *                bf16 roundings of the gate and up products (the bytes of the
 *                unfused product followed by swiglu()); 0: out [numel, 2F].
 * Tables as for grouped_gemm_gate_up (NULL tables: one dense group, E = 1,
 * no sorted_pair). Limits: block_m == 128; H % 128 == 0; F % 128 == 0;
 * 16-byte aligned qa, qw, out. MOE_ERR_INVALID_ARG for inconsistent sizes or
 * tables; MOE_ERR_UNSUPPORTED for block_m != 128, or when a_rows * H or
 * 2F * H (the activation codes, one group's weight codes) reach 2^32 bytes. */
int grouped_gemm_gate_up_fp8(const uint8_t* qa, const float* sa, int64_t a_rows, const int32_t* sorted_pair,
                             int top_k, const uint8_t* qw, const float* sw, const int32_t* group_sizes,
                             const int32_t* group_offsets, const int32_t* group_padded_offsets,
                             const int32_t* group_idx_for_bx, int64_t numel, int E, int H, int F,
                             int padding_m, int block_m, int fuse_swiglu, uint16_t* out,
                             hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H_ */
