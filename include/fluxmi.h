/*
 * fluxmi.h -- C ABI of libfluxmi: tile-granular GEMM fused with the
 * tensor-/expert-parallel data movement around it, for AMD Instinct MI355X
 * (gfx950), one GPU's share of the work.
 *
 * Operators (after the Flux README's five kernels, "快速开始"):
 *   fm_gemm              plain GEMM (the "gemm_only" reference point)
 *   fm_ag_gemm           AllGather fused with GEMM (dense MLP layer 0)
 *   fm_gemm_rs           GEMM fused with ReduceScatter (dense MLP layer 1)
 *   fm_moe_gather_gemm   token gather fused with grouped expert GEMM (MoE layer 0)
 *   fm_moe_gemm_scatter  grouped expert GEMM fused with top-k weighted
 *                        scatter-reduce (MoE layer 1)
 * plus the AllGather variants fm_ag_gemm_pull (chunks read in place),
 * fm_ag_gemm_producers (copies done by workgroups of the same launch),
 * fm_moe_ag_gather_gemm (MoE layer 0 behind a token AllGather) with its
 * producer-workgroup and pull-mode forms (fm_moe_ag_gather_gemm_producers,
 * fm_moe_ag_gather_gemm_pull), the producer
 * half of the chunk-arrival protocol (fm_chunk_push, fm_chunk_push_dma,
 * fm_chunk_signal_paced) and the routing index on its own (fm_moe_route).
 *
 * Conventions for every call:
 *  - All matrices are dense and row-major.  A / X are [M, K]; B / W are [K, N].
 *  - Every pointer argument that names a matrix, flag, index buffer or
 *    workspace is a device pointer to memory owned by the caller; the library
 *    allocates nothing, keeps no state of its own between calls beyond cached
 *    device properties (the compute-unit count), and never synchronizes the
 *    host.  State that must outlive one call (the MoE operators' counters and
 *    completion flags) lives in a caller-owned workspace whose size
 *    fm_moe_workspace_bytes gives.  Calls are enqueued on `stream` (NULL =
 *    the null stream) and return before the work runs; every call is
 *    re-entrant for disjoint buffers.
 *  - 16-bit operands are IEEE binary16 (FM_F16) or bfloat16 (FM_BF16); every
 *    product is accumulated in fp32; narrowing to 16 bits rounds to nearest
 *    even.
 *  - Shape requirements: sizes >= 0; N and K multiples of 8; matrix pointers
 *    16-byte aligned.  A size of 0 in M or N makes the call a no-op; K == 0
 *    yields a zero product.
 *  - Errors: arguments are validated before anything is launched; an invalid
 *    call returns FM_ERR_INVALID_ARG or FM_ERR_UNSUPPORTED and enqueues no
 *    work.  FM_ERR_HIP means the launch itself failed.  A wait that gives up
 *    inside a kernel cannot be returned; it is written to `err_word` instead
 *    (see fm_ag_gemm).  No C++ exception crosses this interface.
 *  - Calls that write the same output on one stream are ordered; calls on
 *    different streams that write the same buffer race.
 *
 * Chunk-arrival protocol (fm_ag_gemm and its variants, fm_moe_ag_gather_gemm):
 *  - A producer makes a chunk's bytes visible device-wide before it publishes
 *    the chunk's flag.  The portable form is a store of the flag with release
 *    semantics at device (agent) scope, as fm_chunk_signal_paced does.  The
 *    library's own copy producers (fm_chunk_push, the producer workgroups of
 *    fm_ag_gemm_producers / fm_moe_ag_gather_gemm_producers) use an equivalent
 *    form that is cheaper on a GPU whose L2 caches are per XCD and not
 *    coherent with each other: each wave writes the chunk with write-through
 *    (system-scope) stores, waits until those stores have completed, passes a
 *    workgroup barrier, and only then updates the counter and the flag with
 *    relaxed atomics.  A release at agent scope would instead write back the
 *    whole L2 of the producer's XCD, once per workgroup.  Any producer must
 *    follow one of these two forms.  Consumers poll with relaxed loads and
 *    acquire at agent scope after the flag is seen.
 *  - The consumers of one launch may occupy every compute unit while they
 *    wait.  A producer kernel that runs on another stream (emulated arrival
 *    on one GPU) must therefore be enqueued on a stream that HIP maps to a
 *    different hardware queue than the consumer's, and before the consumer,
 *    so that its workgroups are dispatched first; with the default four
 *    hardware queues per process, streams created in a row take queues in
 *    turn.  A producer stream that shares the consumer's queue runs after
 *    the consumer, which then waits until spin_limit and reports
 *    FM_ERR_TIMEOUT.  Producers on the copy engines (fm_chunk_push_dma) and
 *    the producer workgroups of the *_producers forms (lowest workgroup ids,
 *    dispatched first) do not depend on this.
 */
#ifndef FLUXMI_H
#define FLUXMI_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fm_status {
    FM_OK = 0,
    FM_ERR_INVALID_ARG = 1,   /* null / misaligned pointer, bad size or count */
    FM_ERR_UNSUPPORTED = 2,   /* dtype combination or size the kernels do not cover */
    FM_ERR_HIP = 3,           /* the HIP launch failed */
    FM_ERR_TIMEOUT = 4        /* only ever written to err_word by a kernel */
} fm_status_t;

typedef enum fm_dtype {
    FM_F16 = 0,
    FM_BF16 = 1,
    FM_F32 = 2
} fm_dtype_t;

/* Activation applied to MoE layer 0's fp32 result before it is rounded and
 * stored (fm_moe_gather_gemm_act). */
typedef enum fm_act {
    FM_ACT_NONE = 0,       /* H = X W1, as fm_moe_gather_gemm */
    FM_ACT_RELU = 1,       /* max(x, 0) */
    FM_ACT_GELU_TANH = 2,  /* x/2 * (1 + tanh(sqrt(2/pi) * (x + 0.044715 x^3))) */
    FM_ACT_SILU = 3        /* x / (1 + exp(-x)) */
} fm_act_t;

/* Library version, major*10000 + minor*100 + patch. */
int fm_version(void);

/* Static, human-readable name of a status code. */
const char* fm_status_str(fm_status_t status);

/*
 * fm_gemm -- C[M,N] = A[M,K] * B[K,N].
 * Defined by the GEMM in the FLUX review's MLP equations (section 三,
 * "MLP 前向传播"); it is also the non-split GEMM that the effective
 * communication time ECT = OverallTime - GEMM_non-split is measured against
 * (same review, "核心公式").
 *   ab   FM_F16 or FM_BF16: element type of A and B.
 *   c    FM_F16, FM_BF16 (same as ab) or FM_F32: element type of C.
 *   A    [M, K] row-major, B [K, N] row-major, C [M, N] row-major (written).
 * C must not overlap A or B.
 */
fm_status_t fm_gemm(fm_dtype_t ab, fm_dtype_t c, int64_t M, int64_t N, int64_t K,
                    const void* A, const void* B, void* C, hipStream_t stream);

/*
 * fm_ag_gemm -- Output1 = GEMM(AllGather(X), W1) with tile-granular overlap
 * (FLUX review, "MLP 前向传播" first GEMM and "AllGather 重叠": the gather and
 * the GEMM are split into tiles and fused in one kernel).
 *   X        [M, K] gathered activation buffer.  Row chunk c = rows
 *            [c*M/n_chunks, (c+1)*M/n_chunks) is written by a producer (a
 *            peer, or fm_chunk_push on another stream) and may be read only
 *            once flags[c] >= epoch.
 *   W        [K, N] weight shard; C [M, N] output (written), dt elements.
 *   n_chunks 1..64, and M % n_chunks == 0.
 *   flags    device array of n_chunks uint32 ready flags.  A producer writes
 *            the chunk, then publishes flags[c] = epoch with release
 *            semantics.  Epochs grow from call to call so flags never need
 *            resetting; the caller zero-fills them once.  In a HIP graph,
 *            whose replays repeat one epoch, zero the flags with a kernel
 *            (not a memset node) at the start of the graph instead.
 *   order    host array of n_chunks chunk indices, the expected arrival order
 *            (e.g. the local chunk first), or NULL for index order.  It only
 *            orders the tiles; the result does not depend on it.
 *   err_word device int32 or NULL.  If a wait exceeds spin_limit polls the
 *            kernel writes FM_ERR_TIMEOUT there, abandons its remaining tiles
 *            (C is then undefined) and exits; the call never hangs.
 *   spin_limit  polls before giving up (each poll sleeps ~0.1 us); 0 selects
 *            the default of 2^24 polls.
 * The result equals fm_gemm on the fully gathered X, bit for bit.
 */
fm_status_t fm_ag_gemm(fm_dtype_t dt, int64_t M, int64_t N, int64_t K, int32_t n_chunks,
                       const void* X, const void* W, void* C,
                       const uint32_t* flags, uint32_t epoch, const int32_t* order,
                       int32_t* err_word, int64_t spin_limit, hipStream_t stream);

/*
 * fm_ag_gemm_pull -- fm_ag_gemm in pull mode (FLUX review, "拉取 vs 推送数据
 * 传输": the compute tiles fetch the communicated data themselves).  No
 * gathered buffer exists: chunk c (rows [c*M/n_chunks, (c+1)*M/n_chunks) of
 * the gathered activation) is read in place from chunks[c], e.g. a peer's
 * buffer mapped into this process, once flags[c] >= epoch.
 *   chunks   host array of n_chunks device pointers, each to a 16-byte
 *            aligned [M/n_chunks, K] row-major block.
 *   W, C, n_chunks, flags, epoch, order, err_word, spin_limit  as fm_ag_gemm.
 * Row tiles are cut per chunk, so no tile reads two buffers; a chunk whose
 * row count is not a multiple of the tile height ends in a partial tile.
 * The result equals fm_gemm on the concatenated chunks, bit for bit.
 */
fm_status_t fm_ag_gemm_pull(fm_dtype_t dt, int64_t M, int64_t N, int64_t K, int32_t n_chunks,
                            const void* const* chunks, const void* W, void* C,
                            const uint32_t* flags, uint32_t epoch, const int32_t* order,
                            int32_t* err_word, int64_t spin_limit, hipStream_t stream);

/*
 * fm_ag_gemm_producers -- fm_ag_gemm with the data movement inside the same
 * launch, on workgroups of its own (COMET article, "COMET 的技术原理": thread
 * blocks are split into communication and computation roles, their ratio
 * adapted to the workload).  The first P workgroups of the grid are
 * producers: for each chunk in `order`, together they copy src[c] into rows
 * [c*M/n_chunks, (c+1)*M/n_chunks) of X and publish flags[c] = epoch
 * (release) once the whole chunk is in.  The other workgroups run the
 * AllGather-GEMM tiles, each after the flags of its chunks.  Producers take
 * the lowest workgroup ids and are dispatched first, so a waiting consumer
 * never holds back the producer it waits for.
 *   src          host array of n_chunks device pointers to [M/n_chunks, K]
 *                source blocks (a peer's chunk); NULL = chunk already in X
 *                (published at the start).  Sources must not overlap X.
 *   X            [M, K] gathered buffer (written by the producers, read by
 *                the consumers).
 *   counters     device uint32 [n_chunks], zero before the first call and
 *                left zero by every call.
 *   n_producers  P, a multiple of 8 (one per XCD per round) up to half the
 *                CUs; 0 picks the largest P that keeps the consumers' tile
 *                waves at their minimum, at most one per MiB copied (the
 *                per-shape choice of the producer:consumer ratio).
 *   W, C, flags, epoch, order, err_word, spin_limit  as fm_ag_gemm.
 * The result equals fm_gemm on the gathered X, bit for bit.
 */
fm_status_t fm_ag_gemm_producers(fm_dtype_t dt, int64_t M, int64_t N, int64_t K,
                                 int32_t n_chunks, const void* const* src, void* X,
                                 const void* W, void* C, uint32_t* flags, uint32_t* counters,
                                 uint32_t epoch, const int32_t* order, int32_t n_producers,
                                 int32_t* err_word, int64_t spin_limit, hipStream_t stream);

/*
 * fm_chunk_signal_paced -- emulated arrival at link speed: publish
 * flags[order[a]] = epoch (release, device scope) once arrive_ns[a]
 * nanoseconds have passed since this call's kernel started, for a = 0 ..
 * n_chunks-1.  The chunk data must already be in place (pull mode, or a
 * pre-filled gathered buffer); only the signals are timed, as a peer's
 * transfer over a link of known bandwidth would deliver them (the review's
 * "拉取 vs 推送数据传输" with the link as the only cost).  One workgroup of one
 * active lane, sleeping between signals, so it takes no measurable compute
 * from a kernel running beside it.
 *   order      host array, a permutation of 0..n_chunks-1, or NULL (index order).
 *   arrive_ns  host array of n_chunks non-decreasing times in [0, 1e9].
 * Times use the device's constant-rate wall clock (hipDeviceAttributeWallClockRate).
 */
fm_status_t fm_chunk_signal_paced(uint32_t* flags, int32_t n_chunks, const int32_t* order,
                                  const int64_t* arrive_ns, uint32_t epoch, hipStream_t stream);

/*
 * fm_chunk_push -- producer side of the chunk-arrival protocol: copy `bytes`
 * from src to dst, then publish *flag = epoch once every byte is visible
 * device-wide (the write-through form of the protocol above: every
 * workgroup's stores have completed before the last one to check in on
 * `counter` stores the flag).  This is what a peer rank's push (the review's
 * "推送模式" in "拉取 vs 推送数据传输") does to this rank's gathered buffer; on
 * one GPU src and dst are both local.
 *   bytes    multiple of 16 (0 = publish the flag only); src/dst 16-byte aligned
 *            and non-overlapping.
 *   counter  device uint32 scratch owned by the caller, zero before the
 *            first call and left zero after every call; one per flag in use.
 *   n_workgroups  copy workgroups, 0 = default (one per 96 KiB, at most
 *                 two per compute unit).
 */
fm_status_t fm_chunk_push(const void* src, void* dst, int64_t bytes, uint32_t* flag,
                          uint32_t* counter, uint32_t epoch, int32_t n_workgroups,
                          hipStream_t stream);

/*
 * fm_chunk_push_dma -- the same producer step on the copy engines: an
 * asynchronous device-to-device copy that uses no compute units, followed on
 * `stream` by a write of epoch into *flag made once the copy has completed.
 * This is how a peer's DMA engine delivers a chunk over a link and then rings
 * the signal (the review's push mode in "拉取 vs 推送数据传输"; the FlagCX
 * guide's put-with-signal), so the consumer's compute units are not spent on
 * the emulated transfer.
 *   bytes  multiple of 16 (0 = write the flag only); src/dst 16-byte aligned
 *          and non-overlapping; flag 4-byte aligned device memory.
 * Returns FM_ERR_HIP if the runtime rejects the copy or the flag write.
 */
fm_status_t fm_chunk_push_dma(const void* src, void* dst, int64_t bytes, uint32_t* flag,
                              uint32_t epoch, hipStream_t stream);

/*
 * fm_gemm_rs -- Output2 = ReduceScatter(GEMM(Output1, W2)), this rank's part
 * (FLUX review, "MLP 前向传播" second GEMM and "ReduceScatter 重叠").
 *   A        [M, K] (K = this rank's shard of the reduction), W [K, N].
 *   dst      host array of n_ranks device pointers; dst[r] is the fp32
 *            [M/n_ranks, N] slice owned by rank r and already holds the other
 *            ranks' partial sums.  The call adds (A*W)[rows of r] into dst[r]
 *            for every r: dst[r] += partial.
 *   n_ranks  1..16, M % n_ranks == 0; rank in [0, n_ranks).
 *            Tiles are taken slice by slice starting at (rank+1) % n_ranks
 *            (the review's tile-coordinate swizzling, "瓦片坐标 Swizzling").
 *   atomic   0: plain read-add-write (this call is the only writer of dst);
 *            1: fp32 atomic adds (several concurrent writers allowed).
 *   dt       FM_F16 or FM_BF16 for A and W.
 */
fm_status_t fm_gemm_rs(fm_dtype_t dt, int64_t M, int64_t N, int64_t K, int32_t n_ranks,
                       int32_t rank, const void* A, const void* W, float* const* dst,
                       int32_t atomic, hipStream_t stream);

/*
 * fm_moe_workspace_bytes -- bytes of device workspace that the MoE operators
 * (fm_moe_route, fm_moe_gather_gemm and its variants, fm_moe_gemm_scatter)
 * need for T tokens with topk pairs each, a hidden size `hidden` and n_local
 * local experts; 0 if the arguments are out of range (T < 0, topk < 1,
 * hidden < 0, n_local outside 1..64).  A workspace of this size serves every
 * call of one MoE layer with these (or smaller) sizes.
 * The workspace is 16-byte aligned device memory owned by the caller.  Fill
 * it with zeros once, before its first use; every call leaves it ready for
 * the next (calls keep an epoch and a few counters in it, so that nothing
 * needs resetting between calls, also when a call is replayed from a HIP
 * graph).  One workspace must not be used by two routes (or two combines) at
 * the same time: issue such calls on one stream, or order their streams.  A
 * route (or layer 0) and a combine may share one workspace concurrently.
 * Separate MoE layers (for instance two expert-parallel ranks emulated on one
 * GPU) that run at the same time need one workspace each.
 */
size_t fm_moe_workspace_bytes(int64_t T, int32_t topk, int64_t hidden, int32_t n_local);

/*
 * fm_moe_route -- expert-sorted row index of this rank's local experts
 * (COMET article, "COMET 的技术原理": the tensor shared between the MoE
 * layers is decomposed along the token dimension).
 *   topk_ids      device int32 [T, topk]: expert of pair p = t*topk + k.
 *   expert_begin  first local expert; local experts are
 *                 [expert_begin, expert_begin + n_local), n_local 1..64.
 *   expert_offsets  device int32 [n_local+1] (written): exclusive prefix sum
 *                 of the local per-expert pair counts.
 *   sorted_pairs  device int32 [T*topk] (written): positions
 *                 [0, expert_offsets[n_local]) hold the local pair ids stably
 *                 sorted by expert (increasing pair id within an expert); the
 *                 rest is left untouched.
 *   ws, ws_bytes  the MoE workspace (fm_moe_workspace_bytes); the per-chunk
 *                 histograms of the counting sort live there.  A null,
 *                 misaligned or too small workspace gives FM_ERR_INVALID_ARG.
 * Deterministic: identical bits on every call.
 */
fm_status_t fm_moe_route(int64_t T, int32_t topk, int32_t expert_begin, int32_t n_local,
                         const int32_t* topk_ids, int32_t* sorted_pairs,
                         int32_t* expert_offsets, void* ws, size_t ws_bytes,
                         hipStream_t stream);

/*
 * fm_moe_gather_gemm -- MoE layer 0 on this rank: route (as fm_moe_route),
 * then for local expert e and its j-th pair p:
 *   H[expert_offsets[e] + j, :] = X[p / topk, :] * W1[e]
 * (Flux README: grouped GEMM of MoE MLP layer 0; the token gather is fused
 * into the GEMM's A loads).  Row counts stay on the device: no host sync.
 *   X   [T, hidden]; W1 [n_local, hidden, ffn]; H [T*topk, ffn] (rows past
 *       expert_offsets[n_local] are left untouched).  dt FM_F16 or FM_BF16.
 *       With hidden = 0 the sum over K is empty: the local rows of H become
 *       0, and X and W1 may be null.  With T = 0 or ffn = 0 only the route
 *       runs.
 *   ws, ws_bytes  the MoE workspace, as fm_moe_route.
 */
fm_status_t fm_moe_gather_gemm(fm_dtype_t dt, int64_t T, int64_t hidden, int64_t ffn,
                               int32_t topk, int32_t expert_begin, int32_t n_local,
                               const void* X, const int32_t* topk_ids, const void* W1,
                               void* H, int32_t* sorted_pairs, int32_t* expert_offsets,
                               void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * fm_moe_gather_gemm_act -- fm_moe_gather_gemm with an activation fused into
 * the epilogue: H[row, :] = act(X[p / topk, :] * W1[e]), the activation taken
 * in fp32 on the accumulated value, then rounded (RNE) to dt.  The FLUX
 * review's MLP forward pass (section 三, "MLP 前向传播") feeds the first GEMM's
 * output to the second as is, which is FM_ACT_NONE; the other forms cover
 * expert MLPs that apply an activation between their two GEMMs.  Arguments,
 * layouts and errors as fm_moe_gather_gemm; an act outside fm_act_t gives
 * FM_ERR_INVALID_ARG before anything is launched.
 */
fm_status_t fm_moe_gather_gemm_act(fm_dtype_t dt, int64_t T, int64_t hidden, int64_t ffn,
                                   int32_t topk, int32_t expert_begin, int32_t n_local,
                                   const void* X, const int32_t* topk_ids, const void* W1,
                                   void* H, int32_t* sorted_pairs, int32_t* expert_offsets,
                                   fm_act_t act, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * fm_moe_ag_gather_gemm -- fm_moe_gather_gemm behind a token AllGather (Flux
 * README: all-gather fused with the grouped GEMM of MoE MLP layer 0): X is
 * the gathered token buffer of n_chunks expert-parallel ranks, chunk c
 * holding tokens [c*T/n_chunks, (c+1)*T/n_chunks), and a tile reads its token
 * rows only after every chunk they come from has flags[c] >= epoch (the
 * protocol of fm_ag_gemm; producers as fm_chunk_push / fm_chunk_push_dma).
 * Rows of an expert are sorted by token, so a tile needs the chunks between
 * its first and last token.  Tiles run in bands of a few M-tiles of one
 * expert, ordered by the expected arrival of the last chunk a band needs, so
 * the rows of the local and earliest chunks start before the others land.
 * topk_ids covers all T tokens and must be complete before the call.
 *   n_chunks  1..64, T % n_chunks == 0; flags device uint32 [n_chunks].
 *   order     host array of n_chunks chunk indices, the expected arrival
 *             order, or NULL for index order (as fm_ag_gemm; it only orders
 *             the tiles).
 *   err_word, spin_limit  as fm_ag_gemm (a wait past the limit writes
 *             FM_ERR_TIMEOUT there; H is then undefined).
 *   ws, ws_bytes  the MoE workspace, as fm_moe_route.
 * The result equals fm_moe_gather_gemm on the fully gathered X, bit for bit.
 */
fm_status_t fm_moe_ag_gather_gemm(fm_dtype_t dt, int64_t T, int64_t hidden, int64_t ffn,
                                  int32_t topk, int32_t expert_begin, int32_t n_local,
                                  const void* X, const int32_t* topk_ids, const void* W1,
                                  void* H, int32_t* sorted_pairs, int32_t* expert_offsets,
                                  int32_t n_chunks, const uint32_t* flags, uint32_t epoch,
                                  const int32_t* order, int32_t* err_word, int64_t spin_limit,
                                  void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * fm_moe_ag_gather_gemm_producers -- fm_moe_ag_gather_gemm with the token
 * AllGather done inside the same launch by producer workgroups (COMET
 * article, "COMET 的技术原理": communication and computation thread blocks
 * of one fused MoE kernel).  The first P workgroups copy src[c] into token
 * rows [c*T/n_chunks, (c+1)*T/n_chunks) of X, chunks taken in `order`, and
 * publish flags[c] = epoch once a chunk is complete; the other workgroups
 * run the layer-0 tiles behind those flags, in the arrival-ordered bands of
 * fm_moe_ag_gather_gemm.  Producers hold the lowest workgroup ids and are
 * dispatched first.
 *   X            [T, hidden] gathered token buffer (written by the producers).
 *   src          host array of n_chunks device pointers to [T/n_chunks, hidden]
 *                blocks; NULL = chunk already in X (published at the start).
 *                Sources are 16-byte aligned and do not overlap X.
 *   counters     device uint32 [n_chunks], zero before the first call and
 *                left zero by every call.
 *   n_producers  P: a multiple of 8, 8 .. half the CUs; 0 = one per ~5 MiB
 *                copied, 8..64.
 *   the rest     as fm_moe_ag_gather_gemm.
 * The result equals fm_moe_gather_gemm on the gathered X, bit for bit.
 */
fm_status_t fm_moe_ag_gather_gemm_producers(
    fm_dtype_t dt, int64_t T, int64_t hidden, int64_t ffn, int32_t topk, int32_t expert_begin,
    int32_t n_local, void* X, const int32_t* topk_ids, const void* W1, void* H,
    int32_t* sorted_pairs, int32_t* expert_offsets, int32_t n_chunks, const void* const* src,
    uint32_t* flags, uint32_t* counters, uint32_t epoch, const int32_t* order,
    int32_t n_producers, int32_t* err_word, int64_t spin_limit, void* ws, size_t ws_bytes,
    hipStream_t stream);

/*
 * fm_moe_ag_gather_gemm_pull -- fm_moe_ag_gather_gemm in pull mode (FLUX
 * review, "拉取 vs 推送数据传输"): no gathered token buffer; each layer-0 tile
 * reads its token rows in place from the owners' chunk buffers (on a node, the
 * peers' activations mapped into this process), after their flags.  Only the
 * tokens routed to this rank's experts are ever read.
 *   chunks  host array of n_chunks device pointers; chunks[c] is the
 *           16-byte aligned [T/n_chunks, hidden] block of tokens
 *           [c*T/n_chunks, (c+1)*T/n_chunks).
 *   the rest  as fm_moe_ag_gather_gemm (flags, epoch, order, err_word,
 *           spin_limit, ws; signals from fm_chunk_signal_paced or a peer).
 * The result equals fm_moe_gather_gemm on the concatenated chunks, bit for
 * bit.
 */
fm_status_t fm_moe_ag_gather_gemm_pull(
    fm_dtype_t dt, int64_t T, int64_t hidden, int64_t ffn, int32_t topk, int32_t expert_begin,
    int32_t n_local, const void* const* chunks, const int32_t* topk_ids, const void* W1, void* H,
    int32_t* sorted_pairs, int32_t* expert_offsets, int32_t n_chunks, const uint32_t* flags,
    uint32_t epoch, const int32_t* order, int32_t* err_word, int64_t spin_limit, void* ws,
    size_t ws_bytes, hipStream_t stream);

/*
 * fm_moe_gemm_scatter -- MoE layer 1 on this rank with the top-k weighted
 * combine fused into the GEMM epilogue (Flux README: grouped GEMM fused with
 * the reduce-scatter of MoE MLP layer 1; COMET article, "COMET 的技术原理":
 * the per-token combine over the experts):
 *   out[t, :] += sum over local pairs p = t*topk + k of
 *                topk_weights[p] * (H[row(p), :] * W2[e(p)])
 * where row(p) is p's position in sorted_pairs (from fm_moe_gather_gemm /
 * fm_moe_route with the same arguments).
 *   H [rows, ffn] with rows = expert_offsets[n_local]; W2 [n_local, ffn, hidden];
 *   topk_weights device fp32 [T, topk]; out device fp32 [T, hidden].  With
 *   ffn = 0 the sum over K is empty (each local pair adds weight x 0) and H
 *   and W2 may be null; with T = 0 or hidden = 0 nothing is launched.
 *   Precondition: the local pairs of one token lie in different experts (a
 *   top-k choice never picks one expert twice).  A token with two pairs in
 *   one local expert is reported as FM_ERR_INVALID_ARG in err_word; the
 *   adds of the row tiles that hold the repeated pair are skipped, and out
 *   is then undefined.
 *   err_word  device int32 or NULL: receives FM_ERR_TIMEOUT if an ordering
 *             wait exceeds spin_limit polls (the launch then abandons its
 *             remaining tiles, out is undefined, the call never hangs), or
 *             FM_ERR_INVALID_ARG as above.  Left untouched otherwise.
 *   spin_limit  polls of one completion flag before giving up (each poll
 *             sleeps ~0.1 us); 0 selects the default of 2^24.
 *   ws, ws_bytes  the MoE workspace (fm_moe_workspace_bytes with the same T,
 *             topk, hidden and n_local or larger); FM_ERR_INVALID_ARG if it
 *             is null, misaligned or too small.
 * The additions into a token row are applied in local-expert order with plain
 * fp32 loads and stores (no atomics), so the result is deterministic.  Each
 * row tile of one expert waits for the tiles of earlier experts in its column
 * whose token ranges overlap its own, through per-(row tile, column tile)
 * completion flags in the workspace, stamped with an epoch that the kernel
 * itself advances there (so the call may be captured in a HIP graph and
 * replayed).  Tiles are handed out by atomic tickets from per-column queues
 * (one per pair of XCDs, each in expert order), so a tile only ever waits for
 * tiles that running workgroups hold: the call completes whatever share of
 * the GPU it gets (another kernel, or another combine on another stream with
 * its own workspace, may run beside it).
 */
fm_status_t fm_moe_gemm_scatter(fm_dtype_t dt, int64_t T, int64_t hidden, int64_t ffn,
                                int32_t topk, int32_t n_local, const void* H, const void* W2,
                                const int32_t* sorted_pairs, const int32_t* expert_offsets,
                                const float* topk_weights, float* out, int32_t* err_word,
                                int64_t spin_limit, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/*
 * fm_moe_gemm_scatter_noalloc -- fm_moe_gemm_scatter for callers that cannot
 * allocate or own a workspace (code under HIP graph capture, tight serving
 * loops, harnesses that forbid device allocation).  The combine's control
 * words and completion flags live in a static device array of the library,
 * 256 KiB per GPU, held until the process ends (its address is looked up, and
 * the array zero-filled by a kernel on `stream`, on the first call on each
 * GPU); the call itself allocates nothing.
 *   Arguments, results and errors as fm_moe_gemm_scatter without (ws,
 *   ws_bytes); the result is bit-identical to it.
 *   Limit: (ceil(T*topk/128) + n_local) * ceil(hidden/128) <= 65216, else
 *   FM_ERR_UNSUPPORTED (the EP=8 workload, T = 16384, top-2, hidden 4096,
 *   8 local experts, needs 8448).  FM_ERR_HIP if the array's address cannot
 *   be obtained.
 *   Every call on one GPU shares that GPU's array: calls that overlap in time
 *   on one GPU (two streams) race and give undefined results; issue them on
 *   one stream, or order the streams.
 */
fm_status_t fm_moe_gemm_scatter_noalloc(fm_dtype_t dt, int64_t T, int64_t hidden, int64_t ffn,
                                        int32_t topk, int32_t n_local, const void* H,
                                        const void* W2, const int32_t* sorted_pairs,
                                        const int32_t* expert_offsets,
                                        const float* topk_weights, float* out,
                                        int32_t* err_word, int64_t spin_limit,
                                        hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FLUXMI_H */
