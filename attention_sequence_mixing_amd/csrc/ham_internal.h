// ham_internal.h -- host-side declarations shared by the C ABI and the kernel
// translation units: argument blocks, workspace layout, launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ham.h"

namespace ham {

// Score partials: every RNN kernel writes, per token and per d_v slice, the
// three sums (p.v, p.p, v.v) of the prediction p = S_{t-1}^T k_t against v_t
// (slices of 16 columns from the token-serial kernel, of 64 from the chunked state
// pass).  The routing kernel adds the slices and forms the cosine.

struct RnnArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* beta;
  const float* g;
  const float* S0;      // [B,H,dk,dv] or null (zeros)
  float* S_out;         // [B,H,dk,dv]
  float* o_rnn32;       // [B,T,H,dv] fp32 (token-serial kernel) or bf16 bits (chunked state
                        // pass, bf16 I/O only), or null (no readout)
  float4* score;        // [B,T,H][slices]
  void* prep;           // chunked path: per-chunk records [B*H][nchunk][kPrepRecordBytes]
  int B, T, H;
  // chunked state pass over segments of the chunk sequence (0: one segment).  Segment p
  // covers chunks [p*seg_chunks, (p+1)*seg_chunks), starts from S0 + p*seg_stride and
  // ends in S_out + p*seg_stride (full pass: only the last segment stores S_out there).
  int seg_chunks;
  size_t seg_stride;
  // chunked full pass, one segment: 0, or 1 (no score partials: the routing scores
  // are the caller's) or 3 (no score partials and the LDS-lean layout that leaves
  // room for an attention workgroup on each CU)
  int variant;
};

// Entering states of the segments of a segmented state pass: S_in[0] = S0 (or 0),
// S_in[p+1] = A_p S_in[p] + B_p, with A_p [dk x dk] and B_p [dk x dv] per head.
struct SegArgs {
  const float* S0;      // [B,H,dk,dv] or null
  const float* A;       // [P-1][B,H,dk,dk]
  const float* Bm;      // [P-1][B,H,dk,dv]
  float* S_in;          // [P][B,H,dk,dv]
  int B, H, P;
};

// Bytes of one chunk record written by the chunked path's prep kernel.
constexpr size_t kPrepRecordBytes = 30720;

struct RouteArgs {
  const float4* score;  // [B,T,H][slices]
  int slices;
  const float* tau;     // [H], or [B,T,H] with tau_per_token
  float* e;             // [B,T,H]
  uint8_t* routed;      // [B,T,H]
  int32_t* chunk_count; // [B*H][nchunk]
  const int32_t* count; // [B,H] entering count (HAM_CONTINUE) or null
  int32_t* count_in;    // [B*H] snapshot of the entering count
  int B, T, H;
  const float* e_in;    // [B,T,H] caller's routing scores (learned router) or null;
                        // when set, score/slices are unused and e is not written
  int tau_per_token;    // tau is [B,T,H] (a threshold schedule along the sequence)
  // block-contiguous routing (blk > 1): whole aligned blocks of blk tokens route
  // on their mean score.  Forward: the call covers whole blocks.  Decode (t_abs
  // set, T = 1): blk_acc [B,H] carries the open block's score sum.
  int blk;
  float* blk_acc;
  const int32_t* t_abs;
  int Hkv;              // KV heads (count, count_in are [B,Hkv]); 0: H
  int e_lds;            // set by the launcher: block routing keeps the scores in LDS
};

struct CompactArgs {
  const void* k;        // attention-path keys   [B,T,H,dk]
  const void* v;        // attention-path values [B,T,H,dv]
  const uint8_t* routed;
  const int32_t* chunk_count;
  const int32_t* count_in;
  void* Kc;             // [B,H,cap,dk]
  void* Vc;             // [B,H,cap,dv]
  int32_t* pos;         // [B,H,cap]
  int32_t* count;       // [B,H] out
  int32_t* ntok;        // [B*H][T] visible-key count per token, or null
  int32_t* status;      // overflow flag or null
  const int32_t* t_abs; // [B] or null
  int t0;
  int B, T, H, cap;
  const float2* rope;   // (cos, sin) of the key rotations, or null: [T][dk/2] rows of the
                        // new tokens (forward), or [B][dk/2] rows at t_abs[b] (decode)
  int blk;              // block-contiguous routing: block size (> 1), else 0
  int Hr;               // RNN heads (routed, chunk_count); H counts the KV heads, each
                        // taking the routing of RNN head h / (H / Hr); 0: H
};

struct StatsArgs {
  const float* e;
  const float* tau;
  const int32_t* chunk_count;
  int32_t* count;       // [B,H]
  int64_t* n_near;      // [H] or null
  float near_band;
  int B, T, H;
  int tau_per_token;    // tau is [B,T,H]
};

struct AttnArgs {
  const void* q;        // attention-path queries [B,T,H,dk]
  const void* Kc;
  const void* Vc;
  const int32_t* ntok;  // [B*H][T]
  const float* o_rnn32; // [B,T,H,dv] fp32, or bf16 bits with ornn_bf16
  const float* gate_rnn;
  const float* gate_kv;
  void* o;
  void* o_rnn;
  void* o_kv;
  float scale;
  float eps;
  int B, T, H, cap;
  const float2* rope;   // [T][dk/2] (cos, sin) of the query rotations, or null
  int ornn_bf16;        // o_rnn32 holds bf16 values (written by the chunked state pass)
  const int32_t* lo;    // [B*H][T] first visible cache entry per query (same-document
                        // masking: keys c in [lo, ntok) are visible), or null (0)
  float* okv32;         // KV heads of another geometry than the RNN's: the attention
                        // readout [B,T,H,dv] fp32 goes here and the mix is left to the
                        // mix kernel (o_rnn32, o, o_rnn, o_kv unused); else null
};

struct DecodeAttnArgs {
  const void* q;        // [B,H,dk]
  const void* Kc;
  const void* Vc;
  const int32_t* count; // [B,H] after the append
  float* part;          // [B*H][nseg][dv + 2]  (acc..., m, l)
  float scale;
  int B, H, cap, seg, nseg;
  const float2* rope;   // [B][dk/2] (cos, sin) of the query rotation at t_abs[b], or null
  const int32_t* lo;    // [B*H] first visible cache entry (same-document masking), or null
};

// Same-document masking: the first cache entry each query may see, the number of
// entries at positions before the query's document start (clamped to the query's
// visible count).  Forward (ntok set): token t of a call starting at t0; decode
// (ntok null, T = 1): the new token, after its append.
struct DocLoArgs {
  const int32_t* doc_start; // [B,T] absolute document start per token
  const int32_t* ntok;      // [B*H][T] visible counts per query, or null (decode)
  const int32_t* count_in;  // [B*H] entries before this call (forward)
  const int32_t* count;     // [B*H] entries after the append (decode; forward with blk)
  const int32_t* pos;       // [B*H][cap] ascending positions
  int32_t* lo;              // [B*H][T] out
  int t0;
  int B, T, H, cap;
  int blk;                  // block-contiguous routing: ntok is not an inclusive count
};

struct DecodeCombineArgs {
  const float* part;
  const int32_t* count;
  const float* o_rnn32;  // [B,H,dv]
  const float* gate_rnn;
  const float* gate_kv;
  void* o;
  void* o_rnn;
  void* o_kv;
  float eps;
  int B, H, seg, nseg;
  float* okv32;          // as AttnArgs::okv32: [B,H,dv] fp32 readout, mix left out
};

// Gated sum of the two headwise-normalised readouts when the KV heads have another
// geometry than the RNN heads: r = Hkv / H KV heads of dv / r columns per RNN head.
struct MixArgs {
  const float* o_rnn32; // [B,T,H,dv] fp32, or bf16 bits with ornn_bf16
  const float* okv32;   // [B,T,Hkv,dv/r] fp32 (the same flat layout)
  const float* gate_rnn;// [B,T,H] or null
  const float* gate_kv; // [B,T,Hkv] or null
  void* o;              // [B,T,H,dv] io dtype
  void* o_rnn;          // [B,T,H,dv] or null
  void* o_kv;           // [B,T,Hkv,dv/r] or null
  float eps;
  int ntok, H, r;       // ntok = B*T
  int ornn_bf16;
};

// Gradients of the attention over the cache (training): the cache and its positions
// as the forward left them, the gradient of the attention readout, and fp32 outputs.
struct AttnBwdArgs {
  const void* q;            // attention-path queries [B,T,H,dk] (io type)
  const void* Kc;           // [B,H,cap,dk]
  const void* Vc;           // [B,H,cap,dv]
  const int32_t* pos;       // [B,H,cap] ascending positions
  const int32_t* count;     // [B,H]
  const int32_t* doc_start; // [B,T] or null
  const float* dO;          // [B,T,H,dv] dL/do_kv
  float* dq;                // [B,T,H,dk]
  float* dKc;               // [B,H,cap,dk] (entries < count)
  float* dVc;               // [B,H,cap,dv]
  float* stat;              // [B,T,H][8] scratch: row maximum, 1/row sum, D, -, lo_t, n_t, -, -
  int2* tile_rng;           // bf16: [B,H,ceil(T/64)] scratch, visible entry range per query tile
  uint16_t* dOh;            // bf16: [B,T,H,dv] scratch, dO = dOh + dOl in bf16 terms
  uint16_t* dOl;
  float scale;
  int B, T, H, cap, t0;
};

// Records msg as this thread's ham_last_error() and returns code (for entry points
// defined outside ham_api.cpp).
int api_fail(int code, const char* msg);

// The host checks of ham_decode_step's dims and arguments, workspace aside: HAM_OK or
// the error code (with its message recorded), as ham_decode_step would return it.
int decode_check(const ham_dims* d, const void* q, const void* k, const void* v, const void* q_attn,
                 const void* k_attn, const void* v_attn, const float* beta, const float* g, const float* tau,
                 const float* block_score, const float* S, const void* Kc, const void* Vc, const int32_t* pos,
                 const int32_t* count, const int32_t* t_abs, const void* o, const void* o_rnn,
                 const void* o_kv, const float* e);

// Gradients of the gated delta-rule RNN: inputs of the forward, dL/do_rnn and
// dL/dS_T; fp32 outputs; scratch for the chunk-start checkpoints and one chunk's
// states per wave.
struct RnnBwdArgs {
  const void* q;        // [B,T,H,dk] io type
  const void* k;
  const void* v;        // [B,T,H,dv]
  const float* beta;    // [B,T,H]
  const float* g;
  const float* S0;      // [B,H,dk,dv] or null
  const float* dO;      // [B,T,H,dv] dL/do_rnn
  const float* dS_T;    // [B,H,dk,dv] or null
  float* dq;            // [B,T,H,dk]
  float* dk;
  float* dv;            // [B,T,H,dv]
  float* dbeta;         // [B,T,H]
  float* dg;
  float* dS0;           // [B,H,dk,dv]
  float* ckpt;          // token-serial reverse, scratch: per wave, the state slab at every chunk start
  float* states;        // token-serial reverse, scratch: per wave, the states of one chunk
  int B, T, H;
  float* scratch;       // chunked reverse: its scratch (rnn_backward_chunked_scratch_floats)
};
size_t rnn_backward_scratch_floats(int B, int H, int T, int dk, int dv);
bool rnn_backward_supported(int dk, int dv);
hipError_t launch_rnn_backward(int io, int dk, int dv, const RnnBwdArgs& a, hipStream_t s);
size_t rnn_backward_chunked_scratch_floats(int B, int H, int T, int dk, int dv);
hipError_t launch_rnn_backward_chunked(int io, int dk, int dv, const RnnBwdArgs& a, hipStream_t s);

// launchers (return hipGetLastError() of the launch)
hipError_t launch_attention_backward(int io, int dk, int dv, const AttnBwdArgs& a, hipStream_t s);
hipError_t launch_rnn_recurrent(int io, int dk, int dv, const RnnArgs& a, hipStream_t s);
hipError_t launch_mix(int io, int dv, const MixArgs& a, hipStream_t s);
int rnn_recurrent_slices(int dv);
// chunked path: prep (per-chunk records, chunks in parallel), then the state pass
hipError_t launch_rnn_chunked_prep(int io, int dk, const RnnArgs& a, hipStream_t s);
hipError_t launch_rnn_chunked_state(int io, int dk, int dv, const RnnArgs& a, hipStream_t s);
// Segmented state pass: mode 0 full (scores, readout when o_rnn32 is set), 1 final
// state only, 2 homogeneous (V = 0, S0 = I, dv = dk: the segment's transition).
hipError_t launch_rnn_chunked_state_seg(int io, int dk, int dv, int mode, int nseg, const RnnArgs& a,
                                        hipStream_t s);
hipError_t launch_seg_combine(int dk, int dv, const SegArgs& a, hipStream_t s);
int rnn_chunked_slices(int dv);
bool rnn_chunked_supported(int io, int dk, int dv);
hipError_t launch_route(const RouteArgs& a, hipStream_t s);
hipError_t launch_compact(int io, int dk, int dv, const CompactArgs& a, hipStream_t s);
hipError_t launch_stats(const StatsArgs& a, hipStream_t s);
hipError_t launch_select_tau(const float* e, int B, int T, int H, long long k, float* tau, hipStream_t s);
hipError_t launch_attention(int io, int dk, int dv, const AttnArgs& a, hipStream_t s);
hipError_t launch_decode_attn(int io, int dk, int dv, const DecodeAttnArgs& a, hipStream_t s);
hipError_t launch_decode_combine(int io, int dv, const DecodeCombineArgs& a, hipStream_t s);
hipError_t launch_rope_table(float2* table, const int32_t* t_abs, int t0, int rows, int dk,
                             double base, hipStream_t s);
hipError_t launch_doc_lo(const DocLoArgs& a, hipStream_t s);

constexpr int kChunk = 64;         // tokens per routing / compaction chunk
constexpr int kDecodeSeg = 1024;   // keys per split-K segment in decode

}  // namespace ham
