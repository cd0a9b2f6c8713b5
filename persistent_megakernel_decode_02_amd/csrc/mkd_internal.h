// Internal declarations shared by the host library and the device code.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "mkd.h"

namespace mkd {

// ---------------------------------------------------------------- schedule spec v4
constexpr int32_t kMagic = 0x314B444D;
constexpr int32_t kVersion = 4;
constexpr int kMaxBatch = 8;  // sequences decoded together
constexpr int kWords = 16;  // words per header and per instruction
enum Opcode : int32_t {
  OP_NOP = 0,
  OP_QKV = 1,         // RMSNorm + [Wq;Wk;Wv] rows (layer 0 also selects the token and embeds it)
  OP_ATTN = 2,        // RoPE + KV append + attention of one q head (one chunk), or of one (kv head, chunk)
  OP_AREDUCE = 3,     // log-sum-exp merge of one q head's chunk partials
  OP_OPROJ = 4,       // Wo rows + residual
  OP_UPGATE = 5,      // RMSNorm + gate/up rows + SiLU product
  OP_DOWN = 6,        // Wd rows + residual
  OP_MOE_UPGATE = 7,  // RMSNorm + router + top-2 + routed experts' gate/up rows + SiLU product
  OP_MOE_DOWN = 8,    // both routed experts' Wd rows, gate-weighted, + residual
  OP_LMHEAD = 9,      // final RMSNorm + LM-head rows, per-tile (max, argmax)
};
// instruction word indices
enum : int { I_OP = 0, I_LAYER, I_STAGE, I_INDEX, I_A, I_B, I_WAIT_STAGE, I_WAIT_COUNT,
             I_WAIT_PREV, I_SIGNAL, I_SEQ };
// header word indices
enum : int { H_MAGIC = 0, H_VERSION, H_NWG, H_NSTAGES, H_MAXINSTR, H_NCHUNKS, H_L, H_D, H_HQ,
             H_HKV, H_HD, H_F, H_V, H_E, H_TOPK, H_BATCH };

struct StageDesc {
  int32_t op, layer, size;  // size: rows (GEMV) or instruction count
};

// host-side schedule helpers (schedule.cpp)
int config_check(const mkd_config* c, const char** why);
void stage_list(const mkd_config* c, int n_chunks, int batch, StageDesc* out, int* n_out, int cap);
int stage_count(const mkd_config* c, int n_chunks);
// blocks stage s may use, and the first of them (the OPROJ stage skips the
// workgroups of the attention stage before it)
void placement(const std::vector<StageDesc>& st, int s, int n_wg, int* avail, int* first);
bool is_tiled(int op);  // stages whose instructions are row tiles
int schedule_build(const mkd_config* c, int n_wg, int n_chunks, int batch, int32_t* out, size_t cap,
                   size_t* n_words, const char** why);
int schedule_validate(const mkd_config* c, const int32_t* w, size_t n, const char** why);

// ---------------------------------------------------------------- device parameters
constexpr int kThreads = 512;  // 8 wavefronts of 64
constexpr int kWaves = kThreads / 64;
constexpr int kPreMax = 16;   // cap on pre_units
constexpr int kFlagAlign = 64;   // per-stage flag arrays start on 256-byte boundaries
constexpr int kTraceWords = 4;   // per instruction: start, inputs ready, end, unused
constexpr int kRed = 256;        // LDS floats reserved for reductions

// weight pointer table layout: global slots, then per-layer slots
constexpr int W_EMBED = 0, W_FINAL_NORM = 1, W_LM_HEAD = 2, W_GLOBAL = 3;
constexpr int WL_ATTN_NORM = 0, WL_Q = 1, WL_K = 2, WL_V = 3, WL_O = 4, WL_FFN_NORM = 5;
constexpr int WL_GATE = 6, WL_UP = 7, WL_DOWN = 8;         // dense
constexpr int WL_ROUTER = 6, WL_EXPERTS = 7;                // MoE: gate[E], up[E], down[E]
inline int layer_slots(const mkd_config* c) { return c->n_experts ? 7 + 3 * c->n_experts : 9; }

// status words (device)
// S_SPEC_HIT / S_SPEC_N: MoE gate/up instructions whose routed expert had been
// predicted (and its first rows staged), out of those that had a prediction
enum : int { S_CODE = 0, S_WG, S_INSTR, S_TOKEN, S_ABORT, S_SPEC_HIT, S_SPEC_N, S_WORDS = 8 };

struct KParams {
  const int32_t* sched;      // schedule words
  const uint64_t* wtab;      // weight pointers
  uint16_t* kv;              // bf16 cache [L][2][hkv][max_seq][hd]
  const float* rope;         // cos [max_seq][hd/2] then sin [max_seq][hd/2]
  // tagged activation buffers: (float value | tag << 32)
  uint64_t* h;               // [d]   residual entering a layer / the LM head
  uint64_t* qkv;             // [qd + 2 kvd]
  uint64_t* part;            // [hq][n_chunks][hd + 2]  (m, l, o[hd])
  uint64_t* aout;            // [qd]
  uint64_t* hmid;            // [d]   residual after attention
  uint64_t* act;             // [top_k * F] (or F)
  uint64_t* route;           // [4]   (expert a, expert b, weight a, weight b)
  uint64_t* lm;              // [2 * n_lm_tiles] (tile max, tile argmax)
  uint32_t* flags;           // [n_stages][flag_stride]: step + 1 once instruction i of a stage is done
  const void* zero;          // >= 1 KiB of readable memory (streamer slots past the end)
  const int32_t* forced;     // [n_steps] or null
  int32_t* tokens_out;       // [n_steps]
  float* logits_out;         // [n_steps][V] or null
  int32_t* status;           // [S_WORDS]
  const int32_t* stop;       // stop word: device address of the caller's pinned host control block
  uint64_t* trace;           // or null
  uint64_t watchdog_ticks;
  int32_t n_wg, max_instr, n_chunks, n_lm_tiles, n_stages, flag_stride;
  int32_t n_steps, max_seq;
  // Batch: B sequences decoded together.  The inputs of row-tiled
  // instructions (h, aout, hmid, act) and the LM-head partials (lm) hold
  // element r of sequence b at word r * B + b; qkv and part, read per
  // sequence by attention, hold sequence b at b * s_qkv (b * s_part); the
  // cache holds sequence b at element b * s_kv.
  int32_t B;
  int32_t first_tok[kMaxBatch];       // token of step 0, per sequence
  int32_t start[kMaxBatch];           // position of step 0, per sequence
  int32_t s_qkv, s_part;              // words
  int64_t s_kv;                       // bf16 elements
  int32_t L, d, hq, hkv, hd, F, V, E, topk, qd, kvd, G, tied, lslots;
  int32_t x_floats;          // LDS floats reserved for the staged input vector
  int32_t out_floats;        // LDS floats for one instruction's GEMV row results
  int32_t res_floats;        // LDS floats for the residual rows of a tile (all sequences)
  int32_t pre_units;         // 1 KiB weight units per wavefront staged in LDS by the
                             // instruction before their own (0 = none): dense gate/up rows
  int32_t pre_off;           // where those units sit: 0 = their own area after the reduction
                             // scratch; else this many floats into the input area, past the
                             // gate/up and O-projection inputs (several sequences)
  int32_t predict;           // MoE: the speculative expert prediction is on
  float eps;
};

size_t lds_bytes(const KParams& p);
// launch the reset kernel and the megakernel (cooperatively, or as a plain
// dispatch of the same grid) on `stream`; ev0/ev1 (may be null) are recorded
// around the megakernel alone
int launch(const KParams& p, size_t ll_words, void* stream, void* ev0, void* ev1, bool cooperative,
           const char** why);
// co-resident workgroups of the persistent kernel for `batch` sequences of a
// dense or MoE model
int max_coop_blocks(int device, size_t lds, int batch, bool moe, int* out);
// The static workspace of mkd_init_static (device address of this device's
// copy; the device must be current)
constexpr size_t kStaticWorkspaceBytes = (size_t)MKD_STATIC_WORKSPACE_BYTES;
int static_workspace(int device, void** ptr, const char** why);
// host-side handles of the persistent kernels (one translation unit each)
const void* kernel_dense();
const void* kernel_moe();
const void* kernel_batch();

}  // namespace mkd
