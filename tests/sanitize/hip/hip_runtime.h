// Host-only stand-in for the HIP runtime header, used only by the sanitized
// host build of the C ABI's validation code (tests/test_sanitized_builds.py):
// gdn_api.cpp and gdn_launch.h need nothing from HIP but the stream handle.
#pragma once
typedef struct ihipStream_t *hipStream_t;
