// Host-sanitizer run of the C ABI's argument validation (built host-only
// with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_sanitizers.py; test infrastructure only).
//
// Every call here fails validation before any device work, so the program
// needs no GPU: invalid configurations, weights and counts, NULL handles and
// outputs, and the status strings. On a machine without a GPU it also takes
// a valid configuration through qmoe_create's failure and clean-up path.
#include <cstdio>
#include <cstring>

#include <hip/hip_runtime_api.h>

#include "../../include/qmoe.h"

static int failures = 0;

#define CHECK(cond, what)                                              \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, what); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

static qmoe_config base_config() {
  qmoe_config c;
  std::memset(&c, 0, sizeof(c));
  c.struct_size = sizeof(qmoe_config);
  c.top_k = 8;
  c.hidden = 2048;
  c.inter = 768;
  c.num_experts = 128;
  c.bits = 4;
  c.block_size = 32;
  c.zero_point = -1;
  c.act_dtype = QMOE_BF16;
  c.normalize_routing = 1;
  c.flags = 0;
  c.max_tokens = 8192;
  return c;
}

// aligned, never dereferenced: validation fails before any use
static const void* const kFake = reinterpret_cast<const void*>(0x10000);

static qmoe_weights fake_weights() {
  qmoe_weights w;
  std::memset(&w, 0, sizeof(w));
  w.fc1_codes = w.fc1_scales = w.fc2_codes = w.fc2_scales = kFake;
  return w;
}

static qmoe_status create(const qmoe_config& c, const qmoe_weights& w, qmoe_handle** h) {
  *h = reinterpret_cast<qmoe_handle*>(0x1234);
  return qmoe_create(&c, &w, 0, h);
}

int main() {
  struct Bad {
    const char* what;
    void (*edit)(qmoe_config&);
    qmoe_status expect;
  };
  const Bad bad[] = {
      {"num_experts 0", [](qmoe_config& c) { c.num_experts = 0; }, QMOE_ERR_INVALID_ARG},
      {"top_k 0", [](qmoe_config& c) { c.top_k = 0; }, QMOE_ERR_INVALID_ARG},
      {"top_k > E", [](qmoe_config& c) { c.top_k = 129; }, QMOE_ERR_INVALID_ARG},
      {"hidden 0", [](qmoe_config& c) { c.hidden = 0; }, QMOE_ERR_INVALID_ARG},
      {"negative inter", [](qmoe_config& c) { c.inter = -768; }, QMOE_ERR_INVALID_ARG},
      {"bits 5", [](qmoe_config& c) { c.bits = 5; }, QMOE_ERR_INVALID_ARG},
      {"block 96", [](qmoe_config& c) { c.block_size = 96; }, QMOE_ERR_INVALID_ARG},
      {"inter not a block multiple", [](qmoe_config& c) { c.inter = 784; }, QMOE_ERR_INVALID_ARG},
      {"zero point 16", [](qmoe_config& c) { c.zero_point = 16; }, QMOE_ERR_INVALID_ARG},
      {"act dtype 7", [](qmoe_config& c) { c.act_dtype = 7; }, QMOE_ERR_INVALID_ARG},
      {"unknown flag", [](qmoe_config& c) { c.flags = 2; }, QMOE_ERR_INVALID_ARG},
      {"negative max_tokens", [](qmoe_config& c) { c.max_tokens = -1; }, QMOE_ERR_INVALID_ARG},
      {"normalize 2", [](qmoe_config& c) { c.normalize_routing = 2; }, QMOE_ERR_INVALID_ARG},
      {"struct size", [](qmoe_config& c) { c.struct_size = 60; }, QMOE_ERR_INVALID_ARG},
      {"huge max_tokens", [](qmoe_config& c) { c.max_tokens = INT64_MAX; }, QMOE_ERR_UNSUPPORTED},
      {"huge hidden", [](qmoe_config& c) { c.hidden = INT64_MAX - 31; }, QMOE_ERR_UNSUPPORTED},
      {"E 2048", [](qmoe_config& c) { c.num_experts = 2048; }, QMOE_ERR_UNSUPPORTED},
      {"top_k 64", [](qmoe_config& c) { c.top_k = 64; }, QMOE_ERR_UNSUPPORTED},
      {"hidden 16384", [](qmoe_config& c) { c.hidden = 16384; }, QMOE_ERR_UNSUPPORTED},
  };
  for (const Bad& b : bad) {
    qmoe_config c = base_config();
    b.edit(c);
    qmoe_handle* h;
    const qmoe_status st = create(c, fake_weights(), &h);
    if (st != b.expect) std::fprintf(stderr, "%s: status %d\n", b.what, static_cast<int>(st));
    CHECK(st == b.expect, b.what);
    CHECK(h == nullptr, "handle not cleared on error");
  }
  {
    qmoe_weights w = fake_weights();
    w.fc1_scales = nullptr;
    qmoe_handle* h;
    CHECK(create(base_config(), w, &h) == QMOE_ERR_INVALID_ARG, "NULL scales accepted");
    w = fake_weights();
    w.fc2_codes = reinterpret_cast<const void*>(0x10004);
    CHECK(create(base_config(), w, &h) == QMOE_ERR_INVALID_ARG, "misaligned codes accepted");
  }
  {
    const qmoe_config c = base_config();
    const qmoe_weights w = fake_weights();
    CHECK(qmoe_create(&c, &w, 0, nullptr) == QMOE_ERR_INVALID_ARG, "NULL out accepted");
    qmoe_handle* h = nullptr;
    CHECK(qmoe_create(nullptr, &w, 0, &h) == QMOE_ERR_INVALID_ARG, "NULL config accepted");
    CHECK(qmoe_create(&c, nullptr, 0, &h) == QMOE_ERR_INVALID_ARG, "NULL weights accepted");
  }
  size_t n = 0, a = 0, b = 0;
  uint32_t bits = 7;
  CHECK(qmoe_destroy(nullptr) == QMOE_OK, "destroy NULL");
  CHECK(qmoe_workspace_size(nullptr, 4, &n) == QMOE_ERR_INVALID_ARG, "workspace_size NULL");
  CHECK(qmoe_forward(nullptr, nullptr, nullptr, nullptr, 4, nullptr, 0, nullptr) == QMOE_ERR_INVALID_ARG,
        "forward NULL");
  CHECK(qmoe_forward_noalloc(nullptr, nullptr, nullptr, nullptr, 4, nullptr) == QMOE_ERR_INVALID_ARG,
        "forward_noalloc NULL");
  CHECK(qmoe_route(nullptr, nullptr, 4, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr) ==
            QMOE_ERR_INVALID_ARG,
        "route NULL");
  CHECK(qmoe_dequant(nullptr, 1, 0, nullptr, nullptr, nullptr) == QMOE_ERR_INVALID_ARG, "dequant NULL");
  CHECK(qmoe_workspace_routing(nullptr, 4, &a, &b) == QMOE_ERR_INVALID_ARG, "workspace_routing NULL");
  CHECK(qmoe_decode_errors(nullptr, nullptr, &bits) == QMOE_ERR_INVALID_ARG, "decode_errors NULL");
  CHECK(qmoe_set_stage_hook(nullptr, nullptr, nullptr) == QMOE_ERR_INVALID_ARG, "stage hook NULL");
  CHECK(std::strcmp(qmoe_status_string(QMOE_OK), "ok") == 0, "status string 0");
  CHECK(std::strcmp(qmoe_status_string(99), "unknown status") == 0,
        "status string 99");
  CHECK(std::strcmp(qmoe_status_string(-1), "unknown status") == 0,
        "status string -1");

  // with no GPU present, a valid configuration fails in the runtime and
  // leaves nothing behind
  int devices = 0;
  if (hipGetDeviceCount(&devices) != hipSuccess || devices == 0) {
    qmoe_handle* h;
    const qmoe_status st = create(base_config(), fake_weights(), &h);
    CHECK(st != QMOE_OK, "create succeeded without a device");
    CHECK(h == nullptr, "handle not cleared after a runtime failure");
  }
  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("abi sanitizer checks passed\n");
  return 0;
}
