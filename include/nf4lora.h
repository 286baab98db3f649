/*
 * nf4lora.h - C ABI of the MI355X (gfx950) frozen-NF4-base LoRA linear and its
 * blockwise weight-streaming pool.
 *
 * Sources (page title, section):
 *   [api]      Poros API reference - "PorosTrainer.from_pretrained" (quantization
 *              "nf4" = 4-bit NF4 QLoRA; lora_rank 16, lora_alpha 32; NF4 reaches
 *              elementwise-exact resident parity), "patch_hf_model" Behavior
 *              (frozen base; blocks of block_size layers; block manager with
 *              cross-stream safety), "Determinism".
 *   [consumer] "Poros on consumer GPUs" - "What you need besides VRAM" (the NF4
 *              base lives in pinned host memory, transferred per block),
 *              "OOM playbook" (block_size never affects parity).
 *   [hn]       HN comment thread on streaming the frozen base (item 49166984),
 *              main comment: the base is read, never written; it sits in host RAM
 *              and streams into a small pool of pre-allocated device buffers,
 *              prefetched one ahead on a dedicated stream.
 *
 * Conventions shared by every entry point:
 *   - Every pointer argument named for a tensor is a DEVICE pointer unless its
 *     comment says host. The caller owns all tensors and both streams; the
 *     library allocates no device memory in any entry point of this header.
 *   - bf16 tensors are passed as uint16_t bit patterns; all matrices are
 *     row-major and densely packed (leading dimension = number of columns).
 *   - Streams are hipStream_t values passed as nf4_stream (NULL = the null
 *     stream). Every compute call only enqueues work on the given stream and
 *     returns; argument errors are detected on the host before anything is
 *     enqueued and are reported synchronously.
 *   - Return value: NF4_OK or a negative NF4_E_* code; nf4_last_error() then
 *     describes the failure (with the offending sizes) for the calling thread.
 *   - Results are deterministic: no atomics, fixed reduction orders, and launch
 *     shapes chosen from the problem sizes alone, so a repeated call returns
 *     bitwise-identical outputs ([api] "Determinism").
 */
#ifndef NF4LORA_H
#define NF4LORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NF4_OK 0
#define NF4_E_ARG (-1)   /* null pointer, bad enum, bad rank */
#define NF4_E_SHAPE (-2) /* sizes that the format or the kernels cannot take */
#define NF4_E_OOM (-3)   /* a pool that does not fit the device slab given */
#define NF4_E_HIP (-4)   /* a HIP runtime call failed */
#define NF4_E_STATE (-5) /* pool call out of order (release without acquire, ...) */
#define NF4_E_BUSY (-6)  /* no pool slot can be reused right now */

#define NF4_BLOCK 64     /* elements per absmax block, along a row */
#define NF4_MAX_RANK 64  /* largest LoRA rank r accepted */

#define NF4_DTYPE_BF16 0
#define NF4_DTYPE_F32 1

typedef void* nf4_stream; /* a hipStream_t */

/* Text of the last error raised on the calling thread ("" if none). */
const char* nf4_last_error(void);

/* ABI version, bumped on any signature change. */
int nf4_abi_version(void);

/*
 * The 16 NF4 levels the library uses, ascending, written to a HOST array.
 * NF4 is QLoRA's 4-bit NormalFloat ([api] "PorosTrainer.from_pretrained",
 * quantization "nf4"): 7 negative and 8 positive N(0,1) quantiles scaled to
 * [-1, 1] plus an exact 0 (index 7). The library derives them itself at load
 * time in extended precision and rounds each once to float32.
 */
int nf4_codebook(float levels_out[16]);

/*
 * Quantise a row-major [rows, cols] matrix to NF4 ([api] quantization "nf4";
 * storage format of [consumer] "What you need besides VRAM").
 *   w       device, rows*cols elements of in_dtype (NF4_DTYPE_BF16 or _F32), finite
 *   codes   device, [rows][cols/2] bytes; element 2i of a row in the low nibble of
 *           byte i, element 2i+1 in the high nibble
 *   absmax  device, [rows][cols/64] float32; absmax of each run of 64 elements
 * Each element gets the nearest level to RN32(w/absmax) (ties to the lower
 * code); an all-zero block gets absmax 0 and code 7. cols % 64 != 0 -> NF4_E_SHAPE.
 * rows == 0 is a no-op.
 */
int nf4_quantize(const void* w, int in_dtype, int64_t rows, int64_t cols,
                 uint8_t* codes, float* absmax, nf4_stream stream);

/*
 * Dequantise to bf16: w[n][k] = RNbf(RN32(level[code] * absmax)) - the exact
 * values every fused kernel below multiplies with.
 *   codes [rows][cols/2], absmax [rows][cols/64] (device, as nf4_quantize writes)
 *   w_bf16 device [rows][cols]
 */
int nf4_dequantize(const uint8_t* codes, const float* absmax, int64_t rows, int64_t cols,
                   uint16_t* w_bf16, nf4_stream stream);

/*
 * Merged dense weight of a LoRA-adapted NF4 linear ([api] "PorosModel.merge_and_unload":
 * the adapters are merged into the base and the module unloaded; the merged weight is
 * kept dense in the model dtype, bf16, not re-quantised):
 *     W_m[n][k] = RNbf( RN32( W[n][k] + RN32(s . l[n][k]) ) ),  l = sum_j B[n][j] A[j][k]
 * with W the dequantised base, s = RN32(alpha / r), l an fp32 sum in rank order
 * (fused multiply-adds). Not on the training path: a one-time export.
 *   codes/absmax  device, the NF4 base W [N][K] (K % 64 == 0)
 *   A             device bf16 [r][K];  B device bf16 [N][r]   (r in 0..NF4_MAX_RANK)
 *   w_out         device bf16 [N][K]  (written; 16-byte aligned)
 * r == 0 writes the dequantised base (A, B may be NULL). Size limits as
 * nf4_lora_linear_fwd (N, K <= 2^21, N*K <= 2^31).
 */
int nf4_merge_lora(const uint8_t* codes, const float* absmax, int64_t N, int64_t K,
                   const uint16_t* A, const uint16_t* B, int r, float alpha,
                   uint16_t* w_out, nf4_stream stream);

/* Bytes of device workspace nf4_lora_linear_fwd needs for these sizes (may be 0). */
size_t nf4_lora_linear_fwd_workspace(int64_t T, int64_t N, int64_t K, int r);

/*
 * Forward of the frozen-NF4-base LoRA linear ([api] "PorosTrainer.from_pretrained":
 * NF4 base with rank-r LoRA; [hn]: the frozen base is only read):
 *     u = x . A^T                          (fp32, saved for the backward)
 *     y = RNbf( x . W^T + s . u . B^T ),   s = RN32(alpha / r), one rounding
 * with W the dequantised base (never materialised: dequantised in registers
 * and fed to bf16 MFMA with fp32 accumulation).
 *   codes/absmax  device, the NF4 base W [N][K] (K % 64 == 0, N % 16 == 0)
 *   x             device bf16 [T][K]
 *   A             device bf16 [r][K];  B device bf16 [N][r]   (r in 0..NF4_MAX_RANK)
 *   y             device bf16 [T][N]  (written)
 *   u_save        device fp32 [T][r]  (written; may be NULL only when r == 0)
 *   ws            device workspace of at least nf4_lora_linear_fwd_workspace()
 *                 bytes, 256-byte aligned (NULL allowed when that size is 0);
 *                 contents on entry are ignored
 * r == 0 computes the base only (A, B, u_save may be NULL). T == 0 is a no-op.
 * Device pointers must be 16-byte aligned. Size limits (NF4_E_SHAPE beyond them,
 * here and in nf4_lora_linear_bwd): N, K <= 2^21, N*K <= 2^31, T <= 2^23.
 */
int nf4_lora_linear_fwd(const uint8_t* codes, const float* absmax, int64_t N, int64_t K,
                        const uint16_t* x, int64_t T,
                        const uint16_t* A, const uint16_t* B, int r, float alpha,
                        uint16_t* y, float* u_save, void* ws, size_t ws_bytes, nf4_stream stream);

/*
 * nf4_lora_linear_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * computation, arguments, limits and errors as nf4_lora_linear_fwd, without the
 * workspace arguments: the workspace is a library-owned device array of
 * NF4_NOALLOC_SCRATCH_BYTES bytes, one per GPU, held from the library's first use on
 * that GPU until the process ends. This call allocates nothing (no hipMalloc, no
 * hipFree, no allocating library routine) and issues no memset; the array keeps the
 * last call's contents, which no call reads before writing.
 * NF4_E_SHAPE when the sizes need more workspace than the array holds
 * (nf4_lora_linear_fwd_workspace() > NF4_NOALLOC_SCRATCH_BYTES; the Qwen2.5
 * 7B/32B/72B projections need at most about 53 MB up to 2048 tokens).
 * Calls that overlap on one GPU (on different streams, or from different host
 * threads) share the array and race: order them on one stream.
 */
#define NF4_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int nf4_lora_linear_fwd_noalloc(const uint8_t* codes, const float* absmax, int64_t N, int64_t K,
                                const uint16_t* x, int64_t T,
                                const uint16_t* A, const uint16_t* B, int r, float alpha,
                                uint16_t* y, float* u_save, nf4_stream stream);

/* Bytes of device workspace nf4_lora_linear_bwd needs for these sizes. */
size_t nf4_lora_linear_bwd_workspace(int64_t T, int64_t N, int64_t K, int r);

/*
 * Backward of the same linear. The base is frozen ([api] "patch_hf_model"
 * Behavior 3; [hn]): no gradient is ever formed for it.
 *     g  = dY . B                          (fp32, in the workspace)
 *     dX = RNbf( dY . W + s . g . A )      one rounding
 *     dA = s . g^T . x                     fp32, overwritten (not accumulated)
 *     dB = s . dY^T . u                    fp32, overwritten
 *   x [T][K], u_save [T][r] (from the forward), dy [T][N]: device
 *   dx  device bf16 [T][K], or NULL to skip dX
 *   dA  device fp32 [r][K], 16-byte aligned; dB device fp32 [N][r] (both may be
 *       NULL when r == 0)
 *   ws  device workspace of at least nf4_lora_linear_bwd_workspace() bytes,
 *       256-byte aligned; its contents on entry are ignored
 * Shapes and r as in the forward. Every output is a fixed-order sum: repeated calls
 * on the same inputs give identical bits.
 */
int nf4_lora_linear_bwd(const uint8_t* codes, const float* absmax, int64_t N, int64_t K,
                        const uint16_t* x, const float* u_save, const uint16_t* dy, int64_t T,
                        const uint16_t* A, const uint16_t* B, int r, float alpha,
                        uint16_t* dx, float* dA, float* dB,
                        void* ws, size_t ws_bytes, nf4_stream stream);

/*
 * Dense-bf16 base variant of the linear ([api] "PorosTrainer.from_pretrained", quantization
 * "bf16_bitwise": an experimental dense-BF16 base streamed blockwise with bitwise resident
 * parity). Same computation, arguments, workspace rules, limits and errors as
 * nf4_lora_linear_fwd / nf4_lora_linear_bwd, with the frozen base given directly as
 *   w   device bf16 [N][K], 16-byte aligned, N*K < 2^30
 * in place of codes + absmax. Every T runs the 128-token kernels (no few-token path).
 */
size_t nf4_lora_linear_fwd_bf16_workspace(int64_t T, int64_t N, int64_t K, int r);
int nf4_lora_linear_fwd_bf16(const uint16_t* w, int64_t N, int64_t K,
                             const uint16_t* x, int64_t T,
                             const uint16_t* A, const uint16_t* B, int r, float alpha,
                             uint16_t* y, float* u_save, void* ws, size_t ws_bytes, nf4_stream stream);
size_t nf4_lora_linear_bwd_bf16_workspace(int64_t T, int64_t N, int64_t K, int r);
int nf4_lora_linear_bwd_bf16(const uint16_t* w, int64_t N, int64_t K,
                             const uint16_t* x, const float* u_save, const uint16_t* dy, int64_t T,
                             const uint16_t* A, const uint16_t* B, int r, float alpha,
                             uint16_t* dx, float* dA, float* dB,
                             void* ws, size_t ws_bytes, nf4_stream stream);

/* ------------------------------------------------------------------ stack glue
 * Elementwise/row kernels of the decoder stack that the streamed base feeds
 * (attention mixing replaced by the identity): h' = h + o(repeat_kv(v(RMSNorm(h)))),
 * h'' = h' + down(SiLU(gate(h_m)) * up(h_m)), h_m = RMSNorm(h'). Tensors are
 * device bf16, row-major, 2-byte aligned; math is fp32 with one bf16 rounding per
 * output; row reductions use a fixed order. Activations are bf16 because that is
 * the model dtype (Poros API reference, "PorosModel.from_pretrained", torch_dtype
 * bfloat16). T == 0 / n == 0 is a no-op.
 */

/* out = RNbf(h * rstd) per row of [T][H], rstd = 1/sqrt(mean(h^2) + eps) (unit
 * gain); rstd (fp32 [T], may be NULL) is saved for the backward. */
int nf4_rmsnorm_fwd(const uint16_t* h, int64_t T, int64_t H, float eps, uint16_t* out, float* rstd,
                    nf4_stream stream);

/* dh = RNbf(dres + rstd*dy - rstd^3 * h * mean(dy*h)) per row; dres (the residual
 * gradient, [T][H]) may be NULL. */
int nf4_rmsnorm_bwd(const uint16_t* h, const float* rstd, const uint16_t* dy, const uint16_t* dres, int64_t T,
                    int64_t H, uint16_t* dh, nf4_stream stream);

/* out = RNbf(a + b + c) over n elements; c may be NULL. out may alias a or b. */
int nf4_add_bf16(const uint16_t* a, const uint16_t* b, const uint16_t* c, int64_t n, uint16_t* out,
                 nf4_stream stream);

/* m = RNbf(SiLU(gate) * up), SiLU(z) = z / (1 + e^-z). */
int nf4_silu_mul_fwd(const uint16_t* gate, const uint16_t* up, int64_t n, uint16_t* m, nf4_stream stream);

/* dgate = RNbf(dm * up * SiLU'(gate)), dup = RNbf(dm * SiLU(gate)). */
int nf4_silu_mul_bwd(const uint16_t* gate, const uint16_t* up, const uint16_t* dm, int64_t n, uint16_t* dgate,
                     uint16_t* dup, nf4_stream stream);

/* a [T][q] from v [T][kv]: each head_dim-wide kv head serves q/kv consecutive
 * query heads (head_dim | kv | q). */
int nf4_repeat_kv_fwd(const uint16_t* v, int64_t T, int64_t q, int64_t kv, int64_t head_dim, uint16_t* a,
                      nf4_stream stream);

/* dv [T][kv] = RNbf(sum over the q/kv query heads of each kv head of da), in head order. */
int nf4_repeat_kv_bwd(const uint16_t* da, int64_t T, int64_t q, int64_t kv, int64_t head_dim, uint16_t* dv,
                      nf4_stream stream);

/*
 * Instrumentation for measurement: the next nf4_lora_linear_fwd or
 * nf4_lora_linear_bwd call made by this host thread records `start` (a
 * hipEvent_t) on its stream immediately before launching its fused
 * dequantise-GEMM kernel and `stop` immediately after it, so
 * hipEventElapsedTime(start, stop) is that one kernel's device time (the
 * small LoRA kernels and any split-K reduction fall outside). The request is
 * consumed by that call. Passing NULL for both cancels a pending request.
 */
int nf4_profile_next_gemm(void* start_event, void* stop_event);

/*
 * Instrumentation: the bf16 MFMA issue rate, for reporting achieved TFLOP/s against a
 * measured ceiling beside the published one. Launches `workgroups` workgroups of 4
 * waves on `stream`; each wave runs `iters` rounds of 8 independent
 * v_mfma_f32_32x32x16_bf16 on register operands (32768 * 8 * iters FLOP per wave) and
 * writes one float to out[4 * workgroup + wave] (device fp32, 4 * workgroups
 * entries, caller-owned). Time it with events on the same stream. NF4_E_ARG for
 * workgroups or iters < 1 or a NULL out.
 */
int nf4_probe_mfma(float* out, int workgroups, int iters, nf4_stream stream);

/*
 * Instrumentation: the HBM read rate of a plain streaming kernel, for reporting the
 * few-token kernels' bytes against a measured read ceiling beside the published one.
 * Launches `workgroups` workgroups of 256 threads on `stream` that read `bytes` bytes
 * of the device buffer `src` (16-byte aligned, bytes a positive multiple of 16) with
 * coalesced 16-byte loads in a grid-stride loop and write the XOR of each thread's
 * 32-bit words to out[256 * workgroup + thread] (device uint32, 256 * workgroups
 * entries, caller-owned; the XOR of all of out is the XOR of all words of src). Time it
 * with events on the same stream. NF4_E_ARG for NULL pointers, misalignment, a size
 * that is not a positive multiple of 16 or workgroups < 1.
 */
int nf4_probe_read(const void* src, size_t bytes, uint32_t* out, int workgroups, nf4_stream stream);

/*
 * The same read probe with `depth` 16-byte loads in flight per thread (4, 8, 16 or 32;
 * nf4_probe_read is depth 8) and, with nontemporal != 0, the loads marked non-temporal
 * (streamed past the caches), so that a sweep over depth and workgroups can show where
 * the read rate stops rising. Arguments and errors as nf4_probe_read, plus NF4_E_ARG for
 * another depth.
 */
int nf4_probe_read_depth(const void* src, size_t bytes, uint32_t* out, int workgroups, int depth,
                         int nontemporal, nf4_stream stream);

/* ------------------------------------------------------------------ stream pool
 * Blockwise residency of the frozen base ([hn] main comment; [api]
 * "patch_hf_model" Behavior 5-6; [consumer] "What you need besides VRAM",
 * "OOM playbook"): the NF4 base of block_size layers at a time lives in a
 * pinned HOST slab; a pool of n_slots device slots (carved from one caller
 * allocation) receives blocks by hipMemcpyAsync on a dedicated copy stream.
 * A block is used on a compute stream between acquire and release; release
 * records an event on that stream, and the copy that later reuses the slot
 * waits on it, so reuse is ordered on the streams, not on the host (which blocks
 * only under a bound on its lead, stream_pool_set_max_ahead).
 * The bytes a kernel sees are the same whether the block is streamed or was
 * copied once (resident), so streamed and resident results are bitwise equal.
 * A pool is used from one host thread at a time.
 */
typedef struct nf4_pool nf4_pool;

typedef struct {
    const void* host; /* pinned host pointer (hipHostMalloc / pin_memory) */
    size_t bytes;     /* bytes of this block; <= slot_bytes */
} nf4_host_block;

typedef struct {
    uint64_t bytes_copied; /* H2D bytes issued */
    uint64_t copies;       /* H2D copies issued */
    uint64_t hits;         /* acquires that found the block already issued/resident */
    uint64_t misses;       /* acquires that had to issue the copy themselves */
    uint64_t evictions;    /* copies that reused a slot holding another block */
} nf4_pool_stats;

/*
 * Create a pool over n_blocks host blocks and n_slots device slots.
 *   blocks       HOST array of n_blocks descriptors (copied; the pinned slabs
 *                must outlive the pool)
 *   device_slab  device memory of at least n_slots * slot_bytes bytes; slot i
 *                starts at device_slab + i * slot_bytes (slot_bytes % 256 == 0)
 *   copy_stream  the dedicated stream for H2D copies (must not be NULL)
 *   out          receives the pool handle
 * NF4_E_OOM if some block is larger than slot_bytes (sizes in the message).
 */
int stream_pool_create(const nf4_host_block* blocks, int n_blocks, void* device_slab,
                       size_t slot_bytes, int n_slots, nf4_stream copy_stream, nf4_pool** out);

/*
 * The current device's pair of streams for a streamed pass ([hn]: blocks are copied
 * on a dedicated stream so that the copies overlap compute): *compute_out for the
 * kernels and the pool's acquire/release, *copy_out for the pool's H2D copies. HIP
 * places a process's streams on a few hardware queues (4 by default), handing them
 * out in creation order; a copy stream that shares the compute stream's queue turns
 * the pool's cross-stream waits into head-of-line blocking there, and copy and
 * compute then run one after the other (measured: 66 ms against 41 ms for 8 blocks
 * of 256 MiB, for every fourth stream created). The two streams are created one right
 * after the other, non-blocking, at the default priority, on the first call for a
 * device, so they take different queues, and are kept until the process ends; later
 * calls return the same pair. Errors: NF4_E_ARG for NULL arguments, NF4_E_HIP if a
 * stream cannot be created.
 */
int stream_pool_streams(nf4_stream* compute_out, nf4_stream* copy_out);

/*
 * Create a pool whose blocks are made of parts, e.g. one pinned host range per layer
 * (a block of block_size layers need not be one contiguous host allocation; [api]
 * "patch_hf_model" Behavior 4: layers regrouped into blocks). Block b is the parts
 * parts[part_begin[b]] .. parts[part_begin[b + 1] - 1], copied back to back into its
 * slot (one hipMemcpyAsync each), so part i starts at the sum of the earlier parts'
 * bytes; every part but a block's last must be a multiple of 256 bytes.
 *   parts       HOST array of part_begin[n_blocks] descriptors (copied; the pinned
 *               ranges must outlive the pool)
 *   part_begin  HOST array of n_blocks + 1 increasing indices, part_begin[0] == 0
 * Other arguments and errors as stream_pool_create (which is this call with one part
 * per block). Each part of a held block can be released on its own
 * (stream_pool_release_part): a later copy into the slot waits only for the release
 * of the parts whose bytes it overwrites.
 */
int stream_pool_create_parts(const nf4_host_block* parts, const int* part_begin, int n_blocks,
                             void* device_slab, size_t slot_bytes, int n_slots, nf4_stream copy_stream,
                             nf4_pool** out);

/*
 * Order in which the parts of a block are copied from now on: ascending (0, the
 * default) or descending (non-zero). A pass that uses a block's parts last to first
 * (a backward pass over layers) sets descending, so that each copy starts with the
 * part whose previous occupant was released first.
 */
int stream_pool_set_order(nf4_pool* pool, int descending);

/*
 * Issue the H2D copy of `block` on the copy stream if it is not already in a
 * slot (no-op then). The victim slot is the least recently used slot not held
 * between acquire and release; the copy first waits for that slot's last
 * release. NF4_E_BUSY when every slot is held.
 */
int stream_pool_prefetch(nf4_pool* pool, int block);

/*
 * Make `block` usable on `compute`: issue its copy if it was not prefetched (a
 * miss), make `compute` wait for the copy, mark the slot held and return its
 * device address in *dev. NF4_E_STATE if the block is already held.
 */
int stream_pool_acquire(nf4_pool* pool, int block, nf4_stream compute, const void** dev);

/*
 * As stream_pool_acquire, but `compute` is made to wait for nothing: before a stream
 * reads part i of the block it must call stream_pool_wait_part(pool, block, i, that
 * stream). With a block copied as several parts (one per layer), the first layers
 * of the block then run while its later parts are still landing ([hn]: copies
 * overlap compute); at the end of a pass, where nothing else is left to overlap,
 * that is what shortens the wait. Errors as stream_pool_acquire.
 */
int stream_pool_acquire_deferred(nf4_pool* pool, int block, nf4_stream compute, const void** dev);

/*
 * Make `stream` wait for the copy of part `part` of a held block (after a deferred
 * acquire; harmless after a plain one). The wait is on an event the copy stream
 * records after that part's copy. NF4_E_STATE if the block is not held; NF4_E_ARG for
 * a part outside the block.
 */
int stream_pool_wait_part(nf4_pool* pool, int block, int part, nf4_stream stream);

/*
 * Bound how far the host may run ahead of the device: with n > 0, every
 * stream_pool_release records an event on its stream and blocks the host until the
 * event recorded n releases earlier has completed (n = 0, the default: no bound).
 * Without a bound a host that issues a whole training step ahead leaves long queues
 * of copies waiting on releases, and the H2D copies behind them were measured to run
 * up to 2x slower (7B stack, 2 slots of 4 layers, one copy per layer: about 2.3 ms per
 * 131 MB layer at first, 2.6-4.6 ms later in the same run; with n = 2 the copies
 * keep their rate). Lowering n waits at once for the marks beyond it. NF4_E_ARG for
 * n < 0.
 */
int stream_pool_set_max_ahead(nf4_pool* pool, int n);

/*
 * End the use of `block` on `compute`: record the last-use events of its parts
 * (those not released by stream_pool_release_part) there. The slot stays valid (a
 * later acquire of the same block is a hit) until a prefetch/acquire of another
 * block reuses it. NF4_E_STATE if not held.
 */
int stream_pool_release(nf4_pool* pool, int block, nf4_stream compute);

/*
 * End the use of one part of a held block on `compute`: record that part's last-use
 * event there. The block stays held; stream_pool_release later records the parts not
 * released this way. NF4_E_STATE if the block is not held or the part was already
 * released during this hold; NF4_E_ARG for a part outside the block.
 */
int stream_pool_release_part(nf4_pool* pool, int block, int part, nf4_stream compute);

/* Counters since creation (HOST struct). */
int stream_pool_stats(const nf4_pool* pool, nf4_pool_stats* out);

/* Which block slot `slot` holds (-1 if none), for tests and tracing. */
int stream_pool_slot_block(const nf4_pool* pool, int slot, int* block_out);

/* Wait for the copy stream to drain, then free the pool's events and state. */
int stream_pool_destroy(nf4_pool* pool);

/*
 * Instrumentation of the copy/compute overlap ([hn]: blocks are prefetched one
 * ahead on a dedicated stream so that copies overlap compute). While enabled, the
 * pool records a pair of timing events around every H2D copy it issues (on the copy
 * stream, after the copy's wait for the slot's last use: the pair spans the copy
 * alone) and around every acquire's wait for a block's copy (on the compute stream:
 * the pair spans the time that stream stood still for the copy; about zero when the
 * prefetch had landed). Whether enabled or not, the pool clocks on the host the time
 * spent inside its own HIP calls (copy issue, event records and waits: a call that
 * blocks the host thread shows there, not in the device spans).
 * stream_pool_timing_collect blocks until the recorded spans have completed, returns
 * their sums and the host clock since the last collect in *out and forgets them.
 * stream_pool_timing_spans (call it before collect, which forgets the spans) blocks
 * likewise and writes up to max_spans of them, copies first in issue order, then
 * acquire waits in issue order, to out (HOST array, caller-owned); *n_out = how many
 * spans are recorded (may exceed max_spans; max_spans = 0 only counts). Device times
 * are ms after the earliest recorded span start, host times ms after that span's
 * issuing call (the two clocks are not synchronised: compare device with device and
 * host with host). NF4_E_ARG for a NULL pool or n_out, a negative max_spans, or a
 * NULL out with max_spans > 0.
 * Enabling adds event records to the streams; it changes no result.
 */
typedef struct {
    double copy_ms;    /* device time of the H2D copies issued while enabled */
    double stall_ms;   /* time the compute streams waited at acquire for a copy */
    uint64_t copies;   /* copies timed */
    uint64_t acquires; /* acquires timed */
    double host_ms;    /* host wall time inside the pool's HIP calls since the last collect */
    double host_max_ms; /* the longest single such call */
    double host_copy_ms;   /* of host_ms: inside hipMemcpyAsync */
    double host_record_ms; /* of host_ms: inside hipEventRecord */
    double host_wait_ms;   /* of host_ms: inside hipStreamWaitEvent */
    double host_sync_ms;   /* of host_ms: blocked in the bound on the host's lead (set_max_ahead) */
} nf4_pool_timing;

#define NF4_SPAN_COPY 0    /* an H2D copy on the copy stream */
#define NF4_SPAN_ACQUIRE 1 /* an acquire's or wait_part's wait on a compute stream */
typedef struct {
    int kind;            /* NF4_SPAN_COPY or NF4_SPAN_ACQUIRE */
    int block;           /* the block copied or acquired */
    int part;            /* the part copied or waited for (index within the block); -1 for an acquire */
    int reserved;
    double start_ms;     /* device: the span's start */
    double end_ms;       /* device: the span's end */
    double host_at_ms;   /* host: when the issuing HIP call began */
    double host_call_ms; /* host: how long that call took */
} nf4_pool_span;

int stream_pool_timing_enable(nf4_pool* pool, int enable);
int stream_pool_timing_collect(nf4_pool* pool, nf4_pool_timing* out);
int stream_pool_timing_spans(nf4_pool* pool, nf4_pool_span* out, int max_spans, int* n_out);

/*
 * Byte layout of one block slab of the streamed base (the slab a pool slot holds;
 * [api] "patch_hf_model" Behavior 4-6: layers regrouped into blocks of block_size;
 * [consumer] "What you need besides VRAM": one slab per block in pinned host
 * memory). For each of `layers` layers in turn and each of the n_proj projections
 * in the order given: NF4 (dense == 0) codes [N][K/2] then absmax [N][K/64] fp32;
 * dense (dense != 0) the bf16 weight [N][K]. Every piece starts at a 256-byte
 * aligned offset, so a layer's bytes are a multiple of 256 and the slab of a block of
 * L layers is the concatenation of L one-layer slabs; streamed and resident runs use
 * the same offsets.
 *   shapes       HOST int64 array of n_proj (N, K) pairs
 *   offsets_out  HOST array of layers * n_proj * 2 size_t, or NULL: entry
 *                [layer][proj][0] = codes (dense: weight) offset, [1] = absmax
 *                offset (0 for dense)
 *   bytes_out    HOST: the slab size
 * NF4_E_ARG for NULL shapes/bytes_out or non-positive counts; NF4_E_SHAPE for an N or
 * K outside 1..2^21 or a K that is not a multiple of 64.
 */
int nf4_block_layout(const int64_t* shapes, int n_proj, int layers, int dense, size_t* offsets_out,
                     size_t* bytes_out);

#ifdef __cplusplus
}
#endif

#endif /* NF4LORA_H */
