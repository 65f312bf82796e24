// Run-time compilation of generated kernels with hiprtc, an on-disk code-object cache, and
// per-device module loading.
#include <dlfcn.h>
#include <hip/hip_runtime_api.h>
#include <hip/hiprtc.h>
#include <sys/stat.h>
#include <unistd.h>

#include <cstdio>
#include <cstdlib>
#include <fstream>
#include <map>
#include <mutex>
#include <sstream>

#include "kernels.hpp"
#include "plan.hpp"

namespace cgtp {

KernelSet::~KernelSet() {
  // Modules are left to process teardown: unloading them here could run after the HIP runtime
  // has shut down (plans destroyed from atexit handlers).
}

std::unique_ptr<KernelSet> make_kernel_set() { return std::unique_ptr<KernelSet>(new KernelSet()); }

static const char* kOptions[] = {
    "--offload-arch=gfx950", "-O3", "-std=c++17",
    // Packed FP32 instructions stay off (v_pk_fma_f32 and friends).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
};
static const int kNumOptions = int(sizeof(kOptions) / sizeof(kOptions[0]));

static uint64_t fnv1a(const std::string& s, uint64_t h = 1469598103934665603ull) {
  for (unsigned char c : s) {
    h ^= c;
    h *= 1099511628211ull;
  }
  return h;
}

static std::string cache_dir() {
  const char* env = std::getenv("CGTP_KERNEL_CACHE");
  if (env && *env) return env;
  Dl_info info;
  if (dladdr(reinterpret_cast<void*>(&cache_dir), &info) && info.dli_fname) {
    std::string so = info.dli_fname;
    size_t slash = so.rfind('/');
    if (slash != std::string::npos) return so.substr(0, slash) + "/kernel_cache";
  }
  return "";
}

static bool read_file(const std::string& path, std::vector<char>* out) {
  std::ifstream f(path, std::ios::binary);
  if (!f) return false;
  out->assign(std::istreambuf_iterator<char>(f), std::istreambuf_iterator<char>());
  return !out->empty();
}

static void write_file_atomic(const std::string& path, const std::vector<char>& data) {
  std::string tmp = path + ".tmp" + std::to_string(getpid());
  {
    std::ofstream f(tmp, std::ios::binary);
    if (!f) return;
    f.write(data.data(), std::streamsize(data.size()));
  }
  std::rename(tmp.c_str(), path.c_str());
}

cgtp_status_t compile_family(Plan& p, const std::string& family, std::string* err) {
  std::lock_guard<std::mutex> lock(p.mu);
  Module& m = p.kernels->families[family];
  if (!m.code.empty()) return CGTP_OK;
  std::string src = generate_source(p, family, err);
  if (src.empty()) return CGTP_ERR_UNSUPPORTED;
  int ver_major = 0, ver_minor = 0;
  hiprtcVersion(&ver_major, &ver_minor);
  std::string tag = src + "|" + std::to_string(ver_major) + "." + std::to_string(ver_minor);
  // The runtime compiler in use is whichever libhiprtc the process bound first (a Python process
  // that imported PyTorch-ROCm first uses the one PyTorch ships): different compilers produce
  // different code for the same source, so the library's path is part of the cache key.
  Dl_info rtc;
  if (dladdr(reinterpret_cast<void*>(&hiprtcCompileProgram), &rtc) && rtc.dli_fname) tag += std::string("|") + rtc.dli_fname;
  for (int k = 0; k < kNumOptions; ++k) tag += std::string("|") + kOptions[k];
  char name[64];
  snprintf(name, sizeof name, "%016llx.co", (unsigned long long)fnv1a(tag));
  std::string dir = cache_dir();
  std::string path = dir.empty() ? "" : dir + "/" + name;
  if (!path.empty() && read_file(path, &m.code)) return CGTP_OK;
  if (std::getenv("CGTP_DUMP_SOURCE")) {
    std::ofstream(std::string(std::getenv("CGTP_DUMP_SOURCE")) + "/" + family + ".hip") << src;
  }
  hiprtcProgram prog;
  if (hiprtcCreateProgram(&prog, src.c_str(), (family + ".hip").c_str(), 0, nullptr, nullptr) != HIPRTC_SUCCESS) {
    *err = "hiprtcCreateProgram failed";
    return CGTP_ERR_COMPILE;
  }
  hiprtcResult rc = hiprtcCompileProgram(prog, kNumOptions, kOptions);
  if (rc != HIPRTC_SUCCESS) {
    size_t n = 0;
    hiprtcGetProgramLogSize(prog, &n);
    std::string log(n, '\0');
    if (n) hiprtcGetProgramLog(prog, &log[0]);
    hiprtcDestroyProgram(&prog);
    *err = "kernel compilation failed for family " + family + ": " + log.substr(0, 4000);
    return CGTP_ERR_COMPILE;
  }
  size_t sz = 0;
  hiprtcGetCodeSize(prog, &sz);
  m.code.resize(sz);
  hiprtcGetCode(prog, m.code.data());
  hiprtcDestroyProgram(&prog);
  if (!path.empty()) {
    mkdir(dir.c_str(), 0755);
    write_file_atomic(path, m.code);
  }
  return CGTP_OK;
}

// ------------------------------------------------------------------ launch timing
// While profiling is on, every launch is bracketed by two HIP events recorded on the launch
// stream; profile_end() waits for them and accumulates the elapsed time per kernel name.
namespace {
std::mutex g_prof_mu;
bool g_prof_on = false;
std::map<hipFunction_t, std::string> g_names;
struct Pending {
  std::string name;
  hipEvent_t a, b;
};
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_event_pool;
std::map<std::string, std::pair<long long, double>> g_totals;  // name -> (launches, ms)

hipEvent_t take_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

void profile_begin() {
  std::lock_guard<std::mutex> lock(g_prof_mu);
  g_prof_on = true;
  g_totals.clear();
}

cgtp_status_t profile_end(std::string* err) {
  std::lock_guard<std::mutex> lock(g_prof_mu);
  g_prof_on = false;
  cgtp_status_t st = CGTP_OK;
  for (auto& p : g_pending) {
    float ms = 0;
    if (hipEventSynchronize(p.b) != hipSuccess || hipEventElapsedTime(&ms, p.a, p.b) != hipSuccess) {
      *err = "hipEventElapsedTime failed";
      st = CGTP_ERR_HIP;
    }
    auto& t = g_totals[p.name];
    t.first += 1;
    t.second += ms;
    g_event_pool.push_back(p.a);
    g_event_pool.push_back(p.b);
  }
  g_pending.clear();
  return st;
}

std::vector<ProfileEntry> profile_entries() {
  std::lock_guard<std::mutex> lock(g_prof_mu);
  std::vector<ProfileEntry> out;
  for (auto& kv : g_totals) out.push_back({kv.first, kv.second.first, kv.second.second});
  return out;
}

cgtp_status_t get_kernel(Plan& p, const std::string& family, const std::string& name, hipFunction_t* f,
                         std::string* err, bool loaded_only) {
  if (!loaded_only) {
    cgtp_status_t st = compile_family(p, family, err);
    if (st != CGTP_OK) return st;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    *err = "hipGetDevice failed";
    return CGTP_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(p.mu);
  Module& m = p.kernels->families[family];
  auto key = std::make_pair(dev, name);
  auto it = m.fns.find(key);
  if (it != m.fns.end()) {
    *f = it->second;
    return CGTP_OK;
  }
  auto mit = m.loaded.find(dev);
  if (mit == m.loaded.end() && loaded_only) {
    *err = "the plan's '" + family + "' kernels are not loaded on device " + std::to_string(dev) +
           ": an allocating call of the same operation must run once on this device first";
    return CGTP_ERR_UNSUPPORTED;
  }
  if (mit == m.loaded.end()) {
    hipModule_t mod;
    hipError_t e = hipModuleLoadData(&mod, m.code.data());
    if (e != hipSuccess) {
      *err = std::string("hipModuleLoadData: ") + hipGetErrorString(e);
      return CGTP_ERR_HIP;
    }
    mit = m.loaded.emplace(dev, mod).first;
  }
  hipFunction_t fn;
  hipError_t e = hipModuleGetFunction(&fn, mit->second, name.c_str());
  if (e != hipSuccess) {
    *err = "hipModuleGetFunction(" + name + "): " + hipGetErrorString(e);
    return CGTP_ERR_HIP;
  }
  m.fns[key] = fn;
  {
    std::lock_guard<std::mutex> plock(g_prof_mu);
    g_names[fn] = name;
  }
  *f = fn;
  return CGTP_OK;
}

cgtp_status_t launch(hipFunction_t f, unsigned grid, unsigned block, unsigned shmem, hipStream_t s, void** args,
                     std::string* err) {
  return launch_grid(f, grid, 1, 1, block, shmem, s, args, err);
}

cgtp_status_t launch_grid(hipFunction_t f, unsigned gx, unsigned gy, unsigned gz, unsigned block, unsigned shmem,
                          hipStream_t s, void** args, std::string* err) {
  if (gx == 0 || gy == 0 || gz == 0) return CGTP_OK;
  hipEvent_t ea = nullptr, eb = nullptr;
  std::string pname;
  {
    std::lock_guard<std::mutex> lock(g_prof_mu);
    if (g_prof_on) {
      ea = take_event();
      eb = take_event();
      auto it = g_names.find(f);
      pname = it == g_names.end() ? "?" : it->second;
    }
  }
  if (ea) (void)hipEventRecord(ea, s);  // timing only: a failed record leaves that launch untimed
  hipError_t e = hipModuleLaunchKernel(f, gx, gy, gz, block, 1, 1, shmem, s, args, nullptr);
  if (eb) {
    (void)hipEventRecord(eb, s);
    std::lock_guard<std::mutex> lock(g_prof_mu);
    g_pending.push_back({pname, ea, eb});
  }
  if (e != hipSuccess) {
    *err = std::string("hipModuleLaunchKernel: ") + hipGetErrorString(e);
    return CGTP_ERR_HIP;
  }
  return CGTP_OK;
}

}  // namespace cgtp
