// Host-side schedule builder and validator (schedule spec v4).
//
// The persistent kernel walks a host-built list of every operation of the
// forward pass (Hyperkernel teardown, "What a megakernel buys"; Kittens VM
// summary, "Method").  The pages fix no format, tiling or assignment; this
// file implements this library's spec v4:
//   a launch decodes B sequences together (batch B >= 1);
//   stages per token: per layer QKV, ATTN, [AREDUCE if n_chunks > 1], OPROJ,
//   UPGATE|MOE_UPGATE, DOWN|MOE_DOWN; then LMHEAD.
//   Row-tiled stage over R rows: n = min(n_wg, R) tiles, tile i = [i*R/n, (i+1)*R/n).
//   ATTN: one chunk -> hq instructions (one q head each); n_chunks > 1 ->
//   hkv * n_chunks (kv_head = i / n_chunks, chunk = i % n_chunks), merged by
//   AREDUCE (hq instructions).  ATTN and AREDUCE repeat that for every
//   sequence: instruction i serves sequence i / n (n per sequence, word
//   I_SEQ) with the operands of instruction i % n.  Row-tiled instructions
//   compute their rows for all B sequences.  Instruction i of a stage runs on block
//   (offset + i) % n_wg; the offset is 0 except for OPROJ, whose tiles skip
//   the blocks that ran the stage before it (ATTN, or AREDUCE) when there
//   are more blocks than that stage has instructions: those blocks finish
//   attention late, and an O-projection tile there would hold the stage up.
#include <string.h>

#include <vector>

#include "mkd_internal.h"

namespace mkd {

bool is_tiled(int op) {
  return op == OP_QKV || op == OP_OPROJ || op == OP_UPGATE || op == OP_DOWN ||
         op == OP_MOE_UPGATE || op == OP_MOE_DOWN || op == OP_LMHEAD;
}

int config_check(const mkd_config* c, const char** why) {
  if (!c) { *why = "null config"; return MKD_E_INVALID; }
  if (c->n_layers < 1) { *why = "n_layers must be >= 1"; return MKD_E_INVALID; }
  if (c->d_model < 8 || c->d_model % 8) { *why = "d_model must be a positive multiple of 8"; return MKD_E_INVALID; }
  if (c->d_ff < 8 || c->d_ff % 8) { *why = "d_ff must be a positive multiple of 8"; return MKD_E_INVALID; }
  if (c->head_dim != 64 && c->head_dim != 128) { *why = "head_dim must be 64 or 128"; return MKD_E_INVALID; }
  if (c->n_kv_heads < 1 || c->n_q_heads < 1 || c->n_q_heads % c->n_kv_heads) {
    *why = "n_q_heads must be a positive multiple of n_kv_heads"; return MKD_E_INVALID;
  }
  if (c->n_q_heads / c->n_kv_heads > 4) { *why = "q heads per kv head must be <= 4"; return MKD_E_INVALID; }
  if (c->vocab < 1) { *why = "vocab must be >= 1"; return MKD_E_INVALID; }
  if (c->n_experts == 0) {
    if (c->top_k != 0) { *why = "top_k must be 0 for a dense FFN"; return MKD_E_INVALID; }
  } else {
    if (c->n_experts < 2 || c->n_experts > 64) { *why = "n_experts must be 0 or in [2, 64]"; return MKD_E_INVALID; }
    if (c->top_k != 2) { *why = "MoE supports top_k == 2"; return MKD_E_INVALID; }
  }
  if (c->tied != 0 && c->tied != 1) { *why = "tied must be 0 or 1"; return MKD_E_INVALID; }
  if (!(c->rms_eps > 0.0f)) { *why = "rms_eps must be > 0"; return MKD_E_INVALID; }
  if (!(c->rope_theta > 1.0)) { *why = "rope_theta must be > 1"; return MKD_E_INVALID; }
  int64_t qd = (int64_t)c->n_q_heads * c->head_dim;
  if (qd % 8) { *why = "n_q_heads * head_dim must be a multiple of 8"; return MKD_E_INVALID; }
  return MKD_OK;
}

int stage_count(const mkd_config* c, int n_chunks) {
  return c->n_layers * (n_chunks > 1 ? 6 : 5) + 1;
}

void stage_list(const mkd_config* c, int n_chunks, int batch, StageDesc* out, int* n_out, int cap) {
  int n = 0;
  auto push = [&](int op, int l, int sz) {
    if (n < cap) out[n] = StageDesc{op, l, sz};
    ++n;
  };
  const int qd = c->n_q_heads * c->head_dim, kvd = c->n_kv_heads * c->head_dim;
  for (int l = 0; l < c->n_layers; ++l) {
    push(OP_QKV, l, qd + 2 * kvd);
    push(OP_ATTN, l, batch * (n_chunks == 1 ? c->n_q_heads : c->n_kv_heads * n_chunks));
    if (n_chunks > 1) push(OP_AREDUCE, l, batch * c->n_q_heads);
    push(OP_OPROJ, l, c->d_model);
    if (c->n_experts) {
      push(OP_MOE_UPGATE, l, c->top_k * c->d_ff);
      push(OP_MOE_DOWN, l, c->d_model);
    } else {
      push(OP_UPGATE, l, c->d_ff);
      push(OP_DOWN, l, c->d_model);
    }
  }
  push(OP_LMHEAD, c->n_layers, c->vocab);
  *n_out = n;
}

static int stage_ninstr(const StageDesc& s, int n_wg) {
  if (is_tiled(s.op)) return s.size < n_wg ? s.size : n_wg;
  return s.size;
}

// blocks stage s may use, and the first of them
void placement(const std::vector<StageDesc>& st, int s, int n_wg, int* avail, int* first) {
  *avail = n_wg;
  *first = 0;
  if (st[s].op == OP_OPROJ && s > 0) {
    const int prev = st[s - 1].size;  // ATTN or AREDUCE instruction count
    if (n_wg > prev) {
      *avail = n_wg - prev;
      *first = prev;
    }
  }
}

static void operands(const StageDesc& s, int n_wg, int n_chunks, int batch, int i, int32_t* a, int32_t* b,
                     int32_t* seq) {
  *seq = 0;
  if (is_tiled(s.op)) {
    const int64_t n = stage_ninstr(s, n_wg), R = s.size;
    *a = (int32_t)(i * R / n);
    *b = (int32_t)((i + 1) * R / n);
    return;
  }
  const int per = s.size / batch;
  *seq = i / per;
  const int j = i % per;
  if (s.op == OP_ATTN) {
    *a = n_chunks == 1 ? j : j / n_chunks;   // q head, or kv head
    *b = n_chunks == 1 ? 0 : j % n_chunks;   // chunk
  } else {  // AREDUCE
    *a = j;
    *b = 0;
  }
}

int schedule_build(const mkd_config* c, int n_wg, int n_chunks, int batch, int32_t* out, size_t cap,
                   size_t* n_words, const char** why) {
  int rc = config_check(c, why);
  if (rc) return rc;
  if (n_wg < 1 || n_wg > 65536) { *why = "n_wg must be in [1, 65536]"; return MKD_E_INVALID; }
  if (n_chunks < 1 || n_chunks > 4096) { *why = "n_chunks must be in [1, 4096]"; return MKD_E_INVALID; }
  if (batch < 1 || batch > kMaxBatch) { *why = "batch must be in [1, 8]"; return MKD_E_INVALID; }
  if (!n_words) { *why = "null n_words"; return MKD_E_INVALID; }
  const int n_st = stage_count(c, n_chunks);
  std::vector<StageDesc> st(n_st);
  int got = 0;
  stage_list(c, n_chunks, batch, st.data(), &got, n_st);
  std::vector<int> cnt(n_st), avail(n_st), first(n_st);
  for (int s = 0; s < n_st; ++s) {
    placement(st, s, n_wg, &avail[s], &first[s]);
    cnt[s] = stage_ninstr(st[s], avail[s]);
  }
  std::vector<int> per_wg(n_wg, 0);
  for (int s = 0; s < n_st; ++s)
    for (int i = 0; i < cnt[s]; ++i) ++per_wg[(first[s] + i) % n_wg];
  int max_instr = 0;
  for (int w = 0; w < n_wg; ++w) max_instr = per_wg[w] > max_instr ? per_wg[w] : max_instr;
  const size_t words = (size_t)kWords + n_wg + (size_t)n_wg * max_instr * kWords;
  *n_words = words;
  if (!out) return MKD_OK;
  if (cap < words) { *why = "output buffer too small for the schedule"; return MKD_E_INVALID; }
  memset(out, 0, words * sizeof(int32_t));
  int32_t* hdr = out;
  hdr[H_MAGIC] = kMagic; hdr[H_VERSION] = kVersion; hdr[H_NWG] = n_wg; hdr[H_NSTAGES] = n_st;
  hdr[H_MAXINSTR] = max_instr; hdr[H_NCHUNKS] = n_chunks; hdr[H_L] = c->n_layers;
  hdr[H_D] = c->d_model; hdr[H_HQ] = c->n_q_heads; hdr[H_HKV] = c->n_kv_heads;
  hdr[H_HD] = c->head_dim; hdr[H_F] = c->d_ff; hdr[H_V] = c->vocab; hdr[H_E] = c->n_experts;
  hdr[H_TOPK] = c->top_k; hdr[H_BATCH] = batch;
  int32_t* counts = out + kWords;
  int32_t* body = counts + n_wg;
  std::vector<int> fill(n_wg, 0);
  for (int s = 0; s < n_st; ++s) {
    const int ws = s == 0 ? n_st - 1 : s - 1;
    for (int i = 0; i < cnt[s]; ++i) {
      const int w = (first[s] + i) % n_wg;
      int32_t* ins = body + ((size_t)w * max_instr + fill[w]++) * kWords;
      ins[I_OP] = st[s].op;
      ins[I_LAYER] = st[s].layer;
      ins[I_STAGE] = s;
      ins[I_INDEX] = i;
      operands(st[s], avail[s], n_chunks, batch, i, &ins[I_A], &ins[I_B], &ins[I_SEQ]);
      ins[I_WAIT_STAGE] = ws;
      ins[I_WAIT_COUNT] = cnt[ws];
      ins[I_WAIT_PREV] = s == 0 ? 1 : 0;
      ins[I_SIGNAL] = s;
    }
  }
  for (int w = 0; w < n_wg; ++w) counts[w] = fill[w];
  return MKD_OK;
}

int schedule_validate(const mkd_config* c, const int32_t* w, size_t n, const char** why) {
  int rc = config_check(c, why);
  if (rc) return rc;
  if (!w || n < (size_t)kWords) { *why = "schedule too short"; return MKD_E_INVALID; }
  if (w[H_MAGIC] != kMagic || w[H_VERSION] != kVersion) { *why = "bad magic/version"; return MKD_E_INVALID; }
  const int n_wg = w[H_NWG], n_st = w[H_NSTAGES], max_instr = w[H_MAXINSTR], n_chunks = w[H_NCHUNKS];
  const int batch = w[H_BATCH];
  if (n_wg < 1 || max_instr < 0 || n_chunks < 1 || batch < 1 || batch > kMaxBatch) {
    *why = "bad header"; return MKD_E_INVALID;
  }
  if (n != (size_t)kWords + n_wg + (size_t)n_wg * max_instr * kWords) { *why = "size mismatch"; return MKD_E_INVALID; }
  if (w[H_L] != c->n_layers || w[H_D] != c->d_model || w[H_HQ] != c->n_q_heads ||
      w[H_HKV] != c->n_kv_heads || w[H_HD] != c->head_dim || w[H_F] != c->d_ff ||
      w[H_V] != c->vocab || w[H_E] != c->n_experts || w[H_TOPK] != c->top_k) {
    *why = "schedule header does not match the config"; return MKD_E_INVALID;
  }
  if (n_st != stage_count(c, n_chunks)) { *why = "stage count"; return MKD_E_INVALID; }
  std::vector<StageDesc> st(n_st);
  int got = 0;
  stage_list(c, n_chunks, batch, st.data(), &got, n_st);
  std::vector<int> cnt(n_st), avail(n_st), first(n_st);
  for (int s = 0; s < n_st; ++s) {
    placement(st, s, n_wg, &avail[s], &first[s]);
    cnt[s] = stage_ninstr(st[s], avail[s]);
  }
  std::vector<std::vector<char>> seen(n_st);
  for (int s = 0; s < n_st; ++s) seen[s].assign(cnt[s], 0);
  const int32_t* counts = w + kWords;
  const int32_t* body = counts + n_wg;
  for (int b = 0; b < n_wg; ++b) {
    if (counts[b] < 0 || counts[b] > max_instr) { *why = "bad per-block count"; return MKD_E_INVALID; }
    int prev = -1;
    for (int j = 0; j < counts[b]; ++j) {
      const int32_t* ins = body + ((size_t)b * max_instr + j) * kWords;
      const int s = ins[I_STAGE];
      if (s < 0 || s >= n_st || ins[I_OP] != st[s].op || ins[I_LAYER] != st[s].layer) {
        *why = "stage/opcode/layer mismatch"; return MKD_E_INVALID;
      }
      if (s < prev) { *why = "a block's list is not in stage order"; return MKD_E_INVALID; }
      prev = s;
      const int i = ins[I_INDEX];
      if (i < 0 || i >= cnt[s] || (first[s] + i) % n_wg != b) { *why = "instruction index or block"; return MKD_E_INVALID; }
      if (seen[s][i]) { *why = "instruction repeated"; return MKD_E_INVALID; }
      seen[s][i] = 1;
      int32_t a, bb, sq;
      operands(st[s], avail[s], n_chunks, batch, i, &a, &bb, &sq);
      if (ins[I_A] != a || ins[I_B] != bb || ins[I_SEQ] != sq) {
        *why = "operands differ from the spec"; return MKD_E_INVALID;
      }
      const int ws = s == 0 ? n_st - 1 : s - 1;
      if (ins[I_WAIT_STAGE] != ws || ins[I_WAIT_COUNT] != cnt[ws] || ins[I_WAIT_PREV] != (s == 0) ||
          ins[I_SIGNAL] != s) {
        *why = "wait/signal fields"; return MKD_E_INVALID;
      }
      for (int k = I_SEQ + 1; k < kWords; ++k)
        if (ins[k] != 0) { *why = "reserved word not zero"; return MKD_E_INVALID; }
    }
  }
  for (int s = 0; s < n_st; ++s)
    for (int i = 0; i < cnt[s]; ++i)
      if (!seen[s][i]) { *why = "an instruction is missing"; return MKD_E_INVALID; }
  return MKD_OK;
}

}  // namespace mkd
