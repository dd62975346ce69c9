// mk_isa.h - instruction encoding, merge-event table and on-chip layout
// shared by the host scheduler (mk_sched.cpp) and the resident interpreter
// (mk_megakernel.hip).
//
// "Inference MegaKernel" (shaojiemike.top), section "hand-written whole-model
// MegaKernel / principle, schedule and dataflow": each compute unit owns a
// queue of fixed-width int32 instructions ([S, Q, 32] in its object table)
// naming the op body and its tile. The page's consumers wait on counters that
// producers bump after a fence. Here every activation a tile consumes carries
// the step's tag in the same 64-bit word as its value, so the wait is on the
// data itself and a step needs neither fences nor counters on its dependency
// edges; counters remain only to elect the one tile that merges split
// attention chunks and the LM-head argmax partials (a "merge event").
#pragma once
#include <stdint.h>

namespace mk {

// op bodies: the page's RMS_NORM is fused into every consumer of a norm
// (QKV, UPGATE, LMHEAD recompute it from the residual stream), RoPE and the
// K/V append live in ATTN, and the O projection with its residual is its own
// body (the page's op list has no O opcode; "residual" is in its op chain).
enum Op : int32_t {
    OP_END = 0,
    OP_QKV = 1,     // rows [r0,r1) of Wqkv . rmsnorm(x_{2l})             -> qkv_l
    OP_ATTN = 2,    // kv head g, tile c of nch: request and K/V blocks split at run time -> a softmax state
    OP_OPROJ = 3,   // rows [r0,r1) of Wo . o_l, plus residual x_{2l}       -> x_{2l+1}
    OP_UPGATE = 4,  // rows [r0,r1) of Wgate, Wup . rmsnorm(x_{2l+1}), SiLU -> act_l
    OP_DOWN = 5,    // rows [r0,r1) of Wdown . act_l, plus residual x_{2l+1} -> x_{2l+2}
    OP_LMHEAD = 6,  // rows [r0,r1) of E . rmsnorm_final(x_{2L}), argmax   -> logits, token
    OP_AMERGE = 7,  // request b, kv head g: merge its tiles' softmax states -> o_l
    OP_COUNT = 8
};

// instruction words
enum : int {
    W_OP = 0,
    W_LAYER = 1,
    W_R0 = 2,
    W_R1 = 3,
    W_B = 4,
    W_G = 5,
    W_C = 6,
    W_NCH = 7,
    W_FLAGS = 8,
    W_MERGE = 9,   // merge event electing the last finisher (-1: none)
    W_SLOT = 10,   // this instruction's slot among the merge's partials
    W_NSLOT = 11,  // slots of the merge
    W_SEQ = 12,    // position in the global topological order
    W_MCTR = 13,   // counter of the merge event (-1: none)
    W_MNEED = 14,  // finishers the merge event waits for
    // operand addresses, bound when the schedule is built (64-bit, low word first):
    W_WA = 16,     // matvec: first weight matrix (UPGATE: gate); LM head: embedding
    W_WB = 18,     // UPGATE: up matrix; else = W_WA
    W_WN = 20,     // norm weight of the op's input (QKV, UPGATE, LM head); else 0
    INSTR_WORDS = 32,
    LDS_INSTR_WORDS = 24  // words of each instruction the interpreter copies into LDS
};

enum : int32_t {
    F_X_FROM_INPUT = 1,  // layer 0: residual stream comes from the embedding row / hidden_in
    F_WRITE_HIDDEN = 2,  // last layer's DOWN: also write hidden_out
    F_STEP_FINAL = 4     // the merge finisher of this instruction ends the step
};

// merge-event table: EV_WORDS int32 per event
enum : int { EV_CTR = 0, EV_NEED = 1, EV_KIND = 2, EV_WORDS = 16 };
enum : int32_t { EVK_MERGE = 1 };
// counters are spaced one 128-byte line apart
constexpr int CTR_STRIDE = 32;

constexpr int WAVE = 64;
constexpr int N_COMPUTE_WAVES = 8;
constexpr int BLOCK_THREADS = N_COMPUTE_WAVES * WAVE;
constexpr int LDS_LIMIT = 160 * 1024;  // gfx950 LDS per workgroup
constexpr int MISC_BYTES = 4096;
constexpr int SLICE_BYTES = 4096;      // weight bytes one wave holds per register slice
constexpr int PREFETCH_SLICES = 2;     // slices each wave keeps in flight
constexpr int ATTN_PART = 64 + 2;      // o[d], m, l of one head
// an attention tile leaves one softmax state per wave and query head in LDS
// before the waves' states are merged
constexpr int attn_state_floats(int G) { return N_COMPUTE_WAVES * G * ATTN_PART; }
constexpr int MAX_B = 8;
// device-clock stamps per instruction in a traced step: start, inputs staged,
// end (merges included), first wave done with its slices, last wave done,
// merge finisher elected, merge inputs gathered, unused
constexpr int TRACE_WORDS = 8;  // MK_TRACE_WORDS of mk.h
enum : int { TR_START = 0, TR_READY = 1, TR_END = 2, TR_FIRST = 3, TR_LAST = 4, TR_ELECT = 5, TR_GATHER = 6 };
constexpr int MAX_G = 8;
// Attention tiles: each kv head has batch x attn_chunks of them, shared out
// over the requests at every step (the attention split of mk_device.h); an
// AMERGE merges one request's tiles, MAX_ATTN_CHUNKS at a time. The split's
// LDS tables hold up to MAX_ATTN_TILES tiles per kv head.
constexpr int MAX_ATTN_CHUNKS = 32;
constexpr int MAX_ATTN_TILES = 128;
// chunks per request the automatic choice gives short K/V (one block per
// wave on half a tile's waves) stops at
constexpr int AUTO_ATTN_CHUNKS = 16;
// attention split modes (mk_schedule_desc::attn_split)
enum : int32_t { SPLIT_BALANCED = 0, SPLIT_PER_REQUEST = 1 };

// device error word: code << 28 | cu << 16 | pc
enum : int32_t { ERR_TIMEOUT = 1, ERR_OPCODE = 2, ERR_RANGE = 3, ERR_NAN = 4 };

}  // namespace mk
