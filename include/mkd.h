/*
 * mkd.h -- C ABI of the persistent batch-1 decode megakernel library (libmkd.so)
 *
 * One cooperative kernel launch decodes N tokens of a pre-norm Llama-style
 * (or Mixtral-style top-2 MoE) decoder at batch 1.  Every workgroup stays
 * resident for the whole launch and walks a host-built instruction list
 * (Kittens VM summary, "Method": one persistent kernel reads an instruction
 * tensor to decide each SM's next work; Hyperkernel teardown, "What a
 * megakernel buys": blocks get a schedule of every operation of the forward
 * pass and synchronise with each other on the device).  The host side only
 * records pointers, builds the schedule and launches (Hyperkernel teardown,
 * "What is in the repository": the host copies tensors where the plan says
 * and launches, without understanding the model; "A single kernel launch,
 * read from the host": one launch per call).
 *
 * Conventions
 *   - Every function returns int: MKD_OK (0) or a negative MKD_E_* code.
 *     Nothing throws across the ABI; mkd_last_error() gives a message for
 *     the calling thread's last failure.
 *   - Pointers marked "device" are GPU memory on the model's device; "host"
 *     pointers are CPU memory.  All memory is the caller's and only
 *     borrowed: weights, KV cache, outputs, a device workspace (sized by
 *     mkd_workspace_bytes; it holds the pointer table, RoPE table, status
 *     words, schedule and tagged activations) and a small pinned host control
 *     block (the stop word).  The library allocates no device or pinned
 *     memory of its own; a handle is a small host object.
 *   - Streams are passed as void* (a hipStream_t; NULL = default stream).
 *   - Functions marked "plumbing" are library housekeeping that no page
 *     describes; every other declaration names the passage it follows.
 */
#ifndef MKD_H
#define MKD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MKD_ABI_VERSION 3

enum {
  MKD_OK = 0,
  MKD_E_INVALID = -1,     /* bad argument, shape, pointer or schedule            */
  MKD_E_HIP = -2,         /* a HIP runtime call failed                           */
  MKD_E_COOPERATIVE = -3, /* the device cannot co-schedule the requested grid    */
  MKD_E_TIMEOUT = -4,     /* mkd_wait: the launch had not finished in time        */
  MKD_E_WATCHDOG = -5,    /* a workgroup waited past the device-side deadline    */
  MKD_E_BOUNDS = -6,      /* a token id or position was out of range on device   */
  MKD_E_NONFINITE = -7,   /* a logit was NaN or infinite                         */
  MKD_E_ABORTED = -8,     /* mkd_abort() stopped the launch                      */
  MKD_E_UNSUPPORTED = -9  /* shape or feature this build does not implement      */
};

/* Model shape.  Pre-norm decoder: RMSNorm -> QKV -> RoPE -> attention ->
 * O-proj + residual -> RMSNorm -> SiLU-gated FFN (or top-k MoE) + residual;
 * final RMSNorm -> LM head.  The model families are the ones the epic-kernel
 * README builds batch-1 megakernels for ("3B model support", "Mixtral 8x7B
 * MoE for batch-1 inference").
 * Limits: d_model % 8 == 0, d_ff % 8 == 0, head_dim in {64, 128},
 * n_q_heads % n_kv_heads == 0 with group <= 4, n_experts in {0} or
 * [2, 64] with top_k == 2, vocab >= 1. */
typedef struct mkd_config {
  int32_t n_layers;
  int32_t d_model;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t d_ff;
  int32_t vocab;
  int32_t n_experts; /* 0 = dense FFN                                   */
  int32_t top_k;     /* 0 for dense, 2 for MoE                          */
  int32_t tied;      /* 1 = LM head is the embedding matrix            */
  float rms_eps;
  float reserved0;
  double rope_theta;
} mkd_config;

/* Device-side outcome of a launch, read by mkd_wait. */
typedef struct mkd_status {
  int32_t code;  /* MKD_OK or the first MKD_E_* the device raised */
  int32_t wg;    /* workgroup that raised it (-1 if none)         */
  int32_t instr; /* index in that workgroup's instruction list     */
  int32_t token; /* decode step                                    */
} mkd_status;

typedef struct mkd_model mkd_model;

/* MKD_ABI_VERSION of the loaded library.  Plumbing. */
int mkd_version(void);

/* Message of the calling thread's last error ("" if none).  The pointer
 * stays valid until the thread's next library call.  Plumbing. */
const char* mkd_last_error(void);

/* Check a configuration against the limits above.  MKD_E_INVALID with a
 * message if it is outside them: the kernels are specialised for these
 * shapes and refuse others, as the released megakernels refuse shapes they
 * were not built for (Hyperkernel teardown, "What is in the repository":
 * one kernel per exact shape, and the host rejects any other). */
int mkd_config_check(const mkd_config* cfg);

/* Number of weight tensors mkd_init expects for cfg (the model is initialised
 * from weight pointers, Hyperkernel teardown, "What is in the repository":
 * the host places each checkpoint tensor where the plan says). */
int mkd_weight_count(const mkd_config* cfg, size_t* n_out);

/* Shape of weight tensor `index` in the fixed pointer order (the plan's
 * tensor map, Hyperkernel teardown, "What is in the repository"):
 *   embed [V, d], final_norm [d], lm_head [V, d] (only when untied), then per
 *   layer attn_norm [d], wq [hq*hd, d], wk [hkv*hd, d], wv [hkv*hd, d],
 *   wo [d, hq*hd], ffn_norm [d], and either w_gate [F, d], w_up [F, d],
 *   w_down [d, F] (dense) or router [E, d], gate_0..gate_{E-1} [F, d],
 *   up_0..up_{E-1} [F, d], down_0..down_{E-1} [d, F] (MoE).
 * All are bf16, row-major ([out, in] for matrices).  cols = 1 for vectors. */
int mkd_weight_shape(const mkd_config* cfg, size_t index, int64_t* rows, int64_t* cols);

/* Bytes of the KV cache for max_seq positions:
 * bf16 [n_layers][2 (K, V)][n_kv_heads][max_seq][head_dim].  Each head's
 * positions are contiguous, so a split-KV chunk is one linear stream (the
 * decode attention the Kittens VM summary's "Results" times). */
int mkd_kv_cache_bytes(const mkd_config* cfg, int32_t max_seq, size_t* bytes_out);

/* Build the instruction tensor (schedule spec v4, one sequence) on the host,
 * without a device.  The spec -- stage order, GEMV row tiling, round-robin block
 * assignment (O-projection tiles skip the blocks that ran attention or its
 * reduction), word layout -- is this library's own; the pages fix none of it
 * (they only say the blocks follow a host-built schedule of every operation,
 * Hyperkernel teardown, "What a megakernel buys").
 * n_wg >= 1 workgroups, n_chunks >= 1 split-KV chunks per KV head.
 * out: host int32 buffer of `capacity` words, or NULL to query the size;
 * *n_words receives the size.  MKD_E_INVALID if capacity is too small. */
int mkd_schedule_build(const mkd_config* cfg, int32_t n_wg, int32_t n_chunks,
                       int32_t* out, size_t capacity, size_t* n_words);

/* As mkd_schedule_build, for `batch` sequences decoded together (1..8): the
 * row-tiled instructions compute their rows for every sequence, attention and
 * its reduction are repeated per sequence (word 10 names it), and header word
 * 15 records the batch.  Each weight is then read once per step for all
 * sequences.  No page describes a batched megakernel; the Kittens VM summary
 * ("Results") quotes a decode figure of a related kernel at a 4-prompt batch. */
int mkd_schedule_build_batch(const mkd_config* cfg, int32_t n_wg, int32_t n_chunks, int32_t batch,
                             int32_t* out, size_t capacity, size_t* n_words);

/* Check a schedule tensor's invariants (ranges, every row of every stage
 * produced exactly once, waits naming the producing stage, lists in stage
 * order): the "barrier that does not deadlock" and "schedule that keeps every
 * SM busy" the Hyperkernel teardown names as the hard parts ("What a
 * megakernel buys").  MKD_OK or MKD_E_INVALID with a message. */
int mkd_schedule_validate(const mkd_config* cfg, const int32_t* words, size_t n_words);

/* Split-KV chunk count the library uses when a schedule leaves it to it
 * (n_chunks = 0): one chunk up to 512 KiB of K and V per KV head at
 * n_positions, else one chunk per workgroup and KV head (at most 64).  The
 * split itself is the decode-attention split of the Kittens VM summary
 * ("Results": a split-KV decode kernel at small batch); the rule is this
 * library's measured choice.  Host only.  MKD_E_INVALID for a bad argument. */
int mkd_default_chunks(const mkd_config* cfg, int32_t n_wg, int32_t n_positions, int32_t* n_chunks);

/* Bytes of device workspace a handle needs to run schedules of n_wg
 * workgroups and n_chunks split-KV chunks (0: mkd_default_chunks at
 * max_seq) for `batch` sequences and positions [0, max_seq).  The host
 * writes its tables to the addresses its plan names inside this memory
 * (Hyperkernel teardown, "What is in the repository").  Host only.
 * MKD_E_INVALID for a bad argument. */
int mkd_workspace_bytes(const mkd_config* cfg, int32_t n_wg, int32_t n_chunks, int32_t batch, int32_t max_seq,
                        size_t* bytes_out);

/* Byte offsets of the workspace regions for the same arguments, into the
 * caller's offsets_out[8]: pointer table, RoPE table, status words, zero
 * page, schedule, tagged activation block, completion flags (inside the
 * activation block), and the total (= mkd_workspace_bytes).  Every region
 * starts on a 256-byte boundary.  Host only; the plan's memory map
 * (Hyperkernel teardown, "What is in the repository"). */
int mkd_workspace_layout(const mkd_config* cfg, int32_t n_wg, int32_t n_chunks, int32_t batch, int32_t max_seq,
                         size_t* offsets_out);

/* Create a model handle on `device` from weight pointers (the host places
 * tensors where the plan says and the model's knowledge stays in the kernel
 * and the plan, Hyperkernel teardown, "What is in the repository").
 * weights: host array of n_weights device pointers (bf16, 16-byte aligned,
 *   order and shapes as in mkd_weight_shape).
 * kv_cache: device, bf16, mkd_kv_cache_bytes(cfg, max_seq) bytes.
 * workspace: device memory of `device`, 256-byte aligned, workspace_bytes
 *   long; at least the tables' part of mkd_workspace_bytes (each schedule
 *   loaded later checks that it fits as a whole).  Init writes the pointer
 *   table, the RoPE cos/sin table (fp64 angles rounded to fp32) for positions
 *   [0, max_seq), the status words and a zero page into it.
 * host_control: pinned host memory mapped for the device (hipHostMalloc, or
 *   a torch tensor made with pin_memory=True), 16 int32 words, 64-byte
 *   aligned; word 0 is the stop word of mkd_abort.  Init zeroes it.
 * Everything is borrowed: the caller keeps it alive until mkd_destroy.
 * Errors: MKD_E_INVALID (shape, null, misaligned or wrong-kind pointer,
 * count, workspace too small), MKD_E_HIP, MKD_E_UNSUPPORTED (device is not
 * gfx950-class or lacks cooperative launch). */
int mkd_init(const mkd_config* cfg, const void* const* weights, size_t n_weights,
             void* kv_cache, int32_t max_seq, void* workspace, size_t workspace_bytes,
             int32_t* host_control, int32_t device, mkd_model** out);

/* As mkd_init, for `batch` sequences (1..8) decoded together by
 * mkd_decode_batch.  kv_cache holds `batch` caches one after the other:
 * batch * mkd_kv_cache_bytes(cfg, max_seq) bytes, sequence b's cache at byte
 * b * mkd_kv_cache_bytes(cfg, max_seq).  Dense models only for batch > 1
 * (MKD_E_UNSUPPORTED for MoE: each sequence would route to its own experts).
 * Schedules built or loaded for the handle must have the same batch.  No
 * page describes a batched megakernel; the Kittens VM summary ("Results")
 * quotes a decode figure of a related kernel at a 4-prompt batch. */
int mkd_init_batch(const mkd_config* cfg, const void* const* weights, size_t n_weights,
                   void* kv_cache, int32_t max_seq, int32_t batch, void* workspace, size_t workspace_bytes,
                   int32_t* host_control, int32_t device, mkd_model** out);

/* Size of the device workspace that mkd_init_static uses: a static array
 * inside the library, one copy per GPU, held until the process ends. */
#define MKD_STATIC_WORKSPACE_BYTES (16u << 20)

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: mkd_init
 * (one sequence) with no workspace argument.  The handle's workspace is the
 * library's static array on `device` (MKD_STATIC_WORKSPACE_BYTES); nothing is
 * allocated, by this call or by the build, load and decode calls on the
 * handle.  The caller still passes weights, KV cache, the pinned host control
 * block and the outputs, as for mkd_init.
 * Limits: the tables and each schedule loaded later must fit in the static
 * size (init: MKD_E_INVALID naming the bytes max_seq needs; schedule build or
 * load: MKD_E_INVALID naming the bytes the schedule needs).  One handle holds
 * a device's array at a time: a second mkd_init_static on the same device
 * fails with MKD_E_INVALID until the first handle is destroyed.  The array
 * keeps the last handle's contents; init rewrites its tables and every launch
 * clears the activations and status first.  Launches on the handle are
 * serialised like any handle's (a second decode while one runs is refused);
 * launches of other processes have their own copy.
 * Errors otherwise as mkd_init. */
int mkd_init_static(const mkd_config* cfg, const void* const* weights, size_t n_weights,
                    void* kv_cache, int32_t max_seq, int32_t* host_control, int32_t device, mkd_model** out);

/* Query the device's compute-unit count and the largest grid a cooperative
 * launch of the megakernel can hold on it: one block per compute unit, all
 * resident at once, as a grid-wide wait requires (Hyperkernel teardown,
 * "What is in the repository": cooperative launches of one block per SM). */
int mkd_device_info(mkd_model* m, int32_t* n_cu, int32_t* max_coop_wg);

/* Host-only query (no device needed): the LDS areas, in floats, that a
 * schedule of n_wg workgroups and n_chunks split-KV chunks for `batch`
 * sequences uses per workgroup on a device with lds_max bytes of LDS per
 * workgroup (0 = unknown: no fitting).  out[6] (caller-owned) receives
 * {input area, row results, residual rows, staged weight units per
 * wavefront (1 KiB each), offset of those units inside the input area
 * (0 = an area of their own after the others), total bytes}.  The staged
 * units are the next instruction's weights loaded ahead of it (epic-kernel
 * README, "L2 prefetching overlapped with prior instructions"), while the
 * workgroup waits out the attention phase: dense gate/up rows (MoE models
 * stage none).
 * MKD_E_INVALID for a bad config or argument. */
int mkd_lds_plan(const mkd_config* cfg, int32_t batch, int32_t n_wg, int32_t n_chunks, int32_t lds_max,
                 int32_t* out);

/* Build (as mkd_schedule_build) and upload the schedule the next launches
 * use into the workspace (the host-built schedule of every operation,
 * Hyperkernel teardown, "What a megakernel buys"); n_wg = 0 means one
 * workgroup per compute unit; n_chunks = 0 takes mkd_default_chunks at the
 * handle's max_seq.  host_out / capacity / n_words as in mkd_schedule_build
 * (host_out may be NULL).  MKD_E_COOPERATIVE if n_wg exceeds what can be
 * co-resident; MKD_E_INVALID if the schedule and its activations do not fit
 * in the handle's workspace. */
int mkd_build_schedule(mkd_model* m, int32_t n_wg, int32_t n_chunks,
                       int32_t* host_out, size_t capacity, size_t* n_words);

/* Upload a schedule built elsewhere (validated first, then as
 * mkd_build_schedule; Hyperkernel teardown, "What a megakernel buys"). */
int mkd_load_schedule(mkd_model* m, const int32_t* words, size_t n_words);

/* Enqueue ONE cooperative launch that decodes n_steps tokens on `stream`
 * (one launch per call, Hyperkernel teardown, "A single kernel launch, read
 * from the host"; the blocks never exit between tokens, "What a megakernel
 * buys").
 * Step i consumes a token at position start_pos + i: first_token for i = 0,
 * otherwise forced_dev[i] when forced_dev is non-NULL and forced_dev[i] >= 0,
 * otherwise the argmax (lowest index on ties) of step i-1's logits.  Step i
 * appends its K and V at position start_pos + i and attends to positions
 * 0 .. start_pos + i of the cache.
 * tokens_out_dev: device int32[n_steps], receives each step's argmax.
 * logits_out_dev: device float[n_steps][vocab] or NULL.
 * forced_dev: device int32[n_steps] or NULL.
 * Asynchronous: returns after enqueueing; use mkd_wait for the outcome.
 * Errors (host-side checks): MKD_E_INVALID (no schedule, first_token not in
 * [0, vocab), start_pos < 0, n_steps < 1, start_pos + n_steps > max_seq,
 * NULL tokens_out_dev, the handle's previous launch still running),
 * MKD_E_COOPERATIVE, MKD_E_HIP.  Clears the stop word before it enqueues. */
int mkd_decode(mkd_model* m, int32_t first_token, int32_t start_pos, int32_t n_steps,
               const int32_t* forced_dev, int32_t* tokens_out_dev, float* logits_out_dev,
               void* stream);

/* Enqueue ONE cooperative launch that decodes n_steps tokens for each of the
 * handle's `batch` sequences together (mkd_init_batch).  Sequence b starts
 * from first_tokens[b] at position start_pos[b] (host arrays of `batch`
 * entries) and proceeds greedily as in mkd_decode; every step reads each
 * weight once for all sequences.
 * tokens_out_dev: device int32[batch][n_steps].
 * logits_out_dev: device float[batch][n_steps][vocab] or NULL.
 * Asynchronous; errors as mkd_decode. */
int mkd_decode_batch(mkd_model* m, const int32_t* first_tokens, const int32_t* start_pos, int32_t n_steps,
                     int32_t* tokens_out_dev, float* logits_out_dev, void* stream);

/* Wait up to timeout_ms (< 0: forever) for the last mkd_decode and read the
 * device status (out may be NULL).  The device-side watchdog (mkd_set_watchdog)
 * ends any wait that outlives its deadline, so a launch cannot hang for good
 * (Hyperkernel teardown, "Hardware fault detection and replanning": a
 * watchdog word, a stop word and bounds flags in a control block, and a host
 * timeout that reports a hang instead of a result).
 * Returns MKD_OK, MKD_E_TIMEOUT (still running), or the device's code:
 * MKD_E_WATCHDOG, MKD_E_BOUNDS, MKD_E_NONFINITE, MKD_E_ABORTED. */
int mkd_wait(mkd_model* m, int32_t timeout_ms, mkd_status* out);

/* Ask the handle's running launch to stop: sets the stop word (word 0 of the
 * host control block).  Workgroup 0 reads it once per decode step; seeing it,
 * it raises the device abort word, which every device-side wait polls, and
 * the launch ends with MKD_E_ABORTED within about one step (Hyperkernel
 * teardown, "Hardware fault detection and replanning": a stop word in the
 * kernel's control block).
 * No effect when no launch is in flight.  mkd_wait and the next launch
 * clear it. */
int mkd_abort(mkd_model* m);

/* Device-side deadline, in milliseconds, for any single wait of a workgroup
 * on another's output (default 2000).  Must be >= 1.  The watchdog word of
 * the control block (Hyperkernel teardown, "Hardware fault detection and
 * replanning"); the launch then ends with MKD_E_WATCHDOG. */
int mkd_set_watchdog(mkd_model* m, int32_t watchdog_ms);

/* Per-instruction timestamps, to account for each opcode's cost (the
 * epic-kernel README's profiling build and its HBM-utilisation plot): when
 * trace_dev is non-NULL, each launch writes,
 * for instruction i of workgroup wg at decode step `step`, four words at
 * trace_dev[((wg * n_steps + step) * max_instr + i) * 4]: wall-clock ticks
 * when the instruction starts, when its inputs are ready, and when it has
 * published its outputs (the fourth word is unused); ticks at mkd_clock_hz.
 * capacity_words must cover n_wg * n_steps * max_instr * 4 at each
 * mkd_decode, else MKD_E_INVALID.  NULL turns tracing off. */
int mkd_set_trace(mkd_model* m, uint64_t* trace_dev, size_t capacity_words);

/* Duration in milliseconds of the last launch's megakernel alone, from HIP
 * events recorded on its stream just before and after the cooperative kernel
 * (the small buffer-reset kernel that precedes it is outside the interval).
 * Call after mkd_wait.  MKD_E_INVALID if nothing has run.  The time that
 * the weight-read floor is set against (Hyperkernel teardown, "Where the
 * numbers sit against the hardware"). */
int mkd_kernel_ms(mkd_model* m, float* ms);

/* Wall-clock tick rate of the device in Hz (for trace and watchdog).
 * Plumbing. */
int mkd_clock_hz(mkd_model* m, double* hz);

/* A plain streaming read of `bytes` (a multiple of 16, at least 16) of
 * device memory at buf_dev, enqueued on `stream` (a hipStream_t, NULL for
 * the default stream) with 16-byte non-temporal loads spread over eight
 * 256-thread workgroups per CU: the HBM read rate the device actually
 * reaches, beside which the decode kernels' fraction of the published peak
 * is read (Hyperkernel teardown, "Where the numbers sit against the
 * hardware": the bytes a kernel must read over the bandwidth bound its time).
 * sink_dev: one device uint32 the kernel may write (it does not in
 * practice).  The caller times it (e.g. with events on the same stream).
 * MKD_E_INVALID for null pointers, a bad size or a buffer not 16-byte
 * aligned, MKD_E_HIP on a launch failure.  Asynchronous. */
int mkd_read_probe(const void* buf_dev, size_t bytes, uint32_t* sink_dev, void* stream);

/* Speculative expert prediction for MoE models (epic-kernel README,
 * "Speculative expert prediction": the top-2 experts are predicted from the
 * pre-attention residual before the router runs, and the predicted experts'
 * weights are loaded early), on (1) or off (0, the default) for launches
 * enqueued after this call.  When on, the workgroup holding a layer's
 * O-projection tile 0 first scores the router on the layer's pre-attention
 * residual and publishes the top two; every O-projection tile followed by a
 * gate/up tile on its workgroup fetches them, and that gate/up tile requests
 * the predicted expert's rows before it waits for its inputs.  The real
 * router always decides: a tile whose routed expert was predicted keeps the
 * requested rows, any other starts again on the routed expert's, so the
 * result never depends on the prediction.  It is off by default because on
 * this part it costs slightly more than it saves (about 0.2-0.5% on the
 * Mixtral shape).  No effect on dense models, or on MoE models with more
 * than 8 experts or d_model above 4096.  MKD_E_INVALID for a null model or
 * `on` other than 0 or 1. */
int mkd_set_expert_prediction(mkd_model* m, int32_t on);

/* Outcome of the expert prediction (mkd_set_expert_prediction) over the last
 * launch mkd_wait saw end.  *predictions: gate/up tiles that had a
 * prediction; *hits: those whose routed expert it named.  Both 0 for dense
 * models and with the prediction off. */
int mkd_spec_stats(mkd_model* m, int32_t* hits, int32_t* predictions);

/* Limits on the per-workgroup LDS plan of schedules built or loaded after
 * this call: the batched input area in floats (0 = no limit; rounded down to
 * whole 512-element segments of every sequence, and never below what the
 * normalised inputs need) and the staged gate/up weight units per wavefront
 * (-1 = no limit).  They only shrink what the plan would use, so that tests
 * can reach the down projection's passes over K on small models and compare
 * staged with unstaged launches; the staging itself is the next
 * instruction's weights loaded ahead of it (epic-kernel README, "L2
 * prefetching overlapped with prior instructions").  MKD_E_INVALID for
 * negative limits (other than -1 for the units). */
int mkd_set_lds_limits(mkd_model* m, int32_t max_input_floats, int32_t max_staged_units);

/* cooperative = 1 (the default): launches are cooperative, so the runtime
 * guarantees the whole grid is resident, as a grid-wide wait needs
 * (Hyperkernel teardown, "What is in the repository").  0: the same grid is
 * dispatched plainly, for profilers that cannot finish their output after a
 * cooperative dispatch; the grid was checked to fit co-resident, so on an
 * idle device it is resident either way.  MKD_E_INVALID otherwise. */
int mkd_set_launch_mode(mkd_model* m, int32_t cooperative);

/* Free the handle (not the borrowed memory).  Waits for an outstanding
 * launch first.  NULL is a no-op.  Plumbing. */
void mkd_destroy(mkd_model* m);

#ifdef __cplusplus
}
#endif

#endif /* MKD_H */
