// Generated gfx950 kernels: source generation (codegen.cpp) and run-time compilation,
// caching and launching (runtime.cpp).
#pragma once

#include <hip/hip_runtime_api.h>

#include <map>
#include <memory>
#include <string>
#include <vector>

#include "cgtp.h"

namespace cgtp {

struct Plan;

// One generated translation unit ("family"): forward, streamed forward, backward, ...
struct Module {
  std::vector<char> code;                       // gfx950 code object
  std::map<int, hipModule_t> loaded;            // per device
  std::map<std::pair<int, std::string>, hipFunction_t> fns;
};

struct KernelSet {
  std::map<std::string, Module> families;
  ~KernelSet();
};

std::unique_ptr<KernelSet> make_kernel_set();

// Kernel source of one family for a plan (deterministic text).
std::string generate_source(const Plan& p, const std::string& family, std::string* err);

// Work decomposition shared by the generator and the launcher.  A task is one wave's share of
// a receiver (or sender): a block of the output (or input) features and 64 channels of it.
struct Task {
  int group;              // output block (forward, receiver backward) or input block (source backward)
  int cb;                 // 64-channel block
  std::vector<int> paths; // paths handled (receiver backward: one register-budgeted subset)
};
// The task lists below are derived from the plan alone; they are built once per plan, on first
// use (every call's host side reads them), and returned by reference.
const std::vector<Task>& forward_tasks(const Plan& p);
const std::vector<Task>& recv_backward_tasks(const Plan& p);
const std::vector<Task>& dbl_recv_tasks(const Plan& p);
const std::vector<Task>& source_tasks(const Plan& p);
// Task groups of a list: tasks sharing a feature block (`group`), in first-appearance order.
// One workgroup runs all channel blocks of a group for one node, so that their waves, which read
// the same coefficient rows edge by edge, share the CU's scalar cache.  `ncb` = the largest
// channel-block count of a group (waves of a smaller group's missing blocks idle).
struct TaskGroups {
  int ncb = 1;
  std::vector<std::vector<int>> tasks;  // per group: task index of channel block cb
};
TaskGroups task_groups(const std::vector<Task>& tasks);
// Waves per (receiver, channel block) in the forward kernels: they deal the edges round-robin.
int fwd_split(const Plan& p);
// Values per edge in the backward's workspace rows: the G row (g_stride values) followed by the
// spherical harmonics Y (sh_dim values), padded to a multiple of 4.
int bwd_row_stride(const Plan& p);
// Receiver-backward edge partials: per task, K phi-bar partials then the Y-bar columns the task's
// paths touch (recv_task_ycols), padded to a multiple of 4; one row of recv_partial_row values
// per edge, tasks in order.
std::vector<int> recv_task_ycols(const Plan& p, const Task& T);
int recv_task_width(const Plan& p, const Task& T);
int recv_partial_row(const Plan& p);
// Values per edge and task written by the receiver backward (phi-bar partials then
// Y-bar partials), padded to a multiple of 4.
int edge_partial_width(const Plan& p);
// Double backward's receiver pass: per task, K phi-bar-dot partials, then the Y-bar-dot and the
// first-order Y-bar columns of the task's Y entries, padded to a multiple of 4; one row of
// dbl_partial_row values per edge in 64-edge tiles (as the first-order backward).
int dbl_task_width(const Plan& p, const Task& T);
int dbl_partial_row(const Plan& p);

struct TaskTables {
  std::vector<Task> fwd, recv, dbl_recv, src;
  int recv_row = 0, dbl_row = 0;
};
const TaskTables& task_tables(const Plan& p);

// Fully connected layout: per output block (receiver side) and input block (source side) the
// state width D (columns (path, q, channel)) and padded row stride ld; per node the sides are
// stored back to back (recv_stride / send_stride elements per node).
struct UvwSideInfo {
  int blk, d, mul, D, ld;
};
struct UvwLayout {
  std::vector<UvwSideInfo> recv, send;
  int n_state_tasks = 0, n_z_tasks = 0;
  int state_acc = 1;  // largest number of state accumulators of a receiver-state task (per lane)
  long long recv_stride = 0, send_stride = 0;
};
UvwLayout uvw_layout(const Plan& p);
// Waves splitting one receiver's edge list in the fully connected state and edge kernels.
constexpr int kMaxStripes = 4;
// The S-bar GEMM of an output block of at most 64 channels (its whole depth) keeps the 64-row
// panel of m-bar in LDS and sweeps kSbarPanelTiles column tiles of 64 per workgroup.
constexpr int kSbarPanelTiles = 8;
inline bool sbar_panel(int mul) { return mul <= 64; }

// Compile (once) and fetch a kernel of a family on the current device.
// loaded_only: fetch only from a module already loaded on the current device (no compilation, no
// module load, hence no device allocation); UNSUPPORTED otherwise.
cgtp_status_t get_kernel(Plan& p, const std::string& family, const std::string& name, hipFunction_t* f,
                         std::string* err, bool loaded_only = false);
cgtp_status_t compile_family(Plan& p, const std::string& family, std::string* err);

// Launch timing (see cgtp_profile_begin in cgtp.h).
struct ProfileEntry {
  std::string name;
  long long launches;
  double ms;
};
void profile_begin();
cgtp_status_t profile_end(std::string* err);
std::vector<ProfileEntry> profile_entries();

// Launch helper: args is an array of pointers to the kernel arguments.
cgtp_status_t launch(hipFunction_t f, unsigned grid, unsigned block, unsigned shmem, hipStream_t s,
                     void** args, std::string* err);
// Three-dimensional grid (also timed by the launch profiler).
cgtp_status_t launch_grid(hipFunction_t f, unsigned gx, unsigned gy, unsigned gz, unsigned block, unsigned shmem,
                          hipStream_t s, void** args, std::string* err);

}  // namespace cgtp
