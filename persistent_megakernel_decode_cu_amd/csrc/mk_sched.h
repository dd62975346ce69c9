// mk_sched.h - host scheduler: tile DAG, events, per-CU queues (no HIP).
#pragma once
#include <cstdint>
#include <string>
#include <vector>

#include "mk.h"
#include "mk_isa.h"

namespace mk {

// Records the thread's last error text and returns `code`.
int set_error(int code, const std::string &msg);

struct Plan {
    mk_config cfg{};
    mk_schedule_desc desc{};
    int n_cus = 0, Q = 0, n_instr = 0, n_events = 0, n_counters = 0;
    int attn_chunks = 0;
    int max_kv_len = 0;
    // LDS layout of a resident workgroup (bytes): misc | instruction queue |
    // residual rows | activation area (matvec inputs, attention staging and
    // rounds, merge staging) | norm weights
    int queue_off = 0, xrow_off = 0, act_off = 0, nw_off = 0, lds_bytes = 0;
    int xrow_stride = 0, act_stride = 0;  // floats per request
    int n_lm_slots = 0;        // LM-head tiles (partial argmax slots)
    std::vector<int32_t> queue;   // [n_cus, Q, INSTR_WORDS]
    std::vector<int32_t> events;  // [n_events, EV_WORDS]
    int64_t stream_max_cu = 0, stream_total = 0;
    int launches = 0;
};

// Shape checks shared by mk_create and the planner.
int check_config(const mk_config &cfg);

int build_plan(const mk_config &cfg, const mk_schedule_desc &desc, Plan &out);

// Number of kernel launches of one unfused step.
int unfused_launches(const mk_config &cfg);

}  // namespace mk
